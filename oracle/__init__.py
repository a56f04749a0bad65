"""CPU oracle for MoE dispatch/combine -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may import this
package.  The product path (``combine_quant_amd``) never does, and the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain single-threaded C, one IEEE binary32
operation per written float operation); this module only marshals numpy arrays through
ctypes.  Function-level citations of the pages are in the C source.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


class OracleCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "W", "E", "BS", "H", "K", "quant_mode", "zero_expert_num", "copy_expert_num",
        "expert_token_nums_type", "mask_kind", "out_dtype", "scales_kind", "scale_format",
        "token_dtype")]

# token element types (x, ori_x, expert outputs, y)
TOKEN_BF16, TOKEN_F16 = 0, 1

# element types of expand_x (out_dtype values; 0 selects the quant mode's default)
CODE_BF16, CODE_INT8, CODE_E4M3, CODE_E5M2, CODE_E2M1 = 0, 1, 2, 3, 4


def _load():
    global _lib
    if _lib is None:
        # MOE_ORACLE_LIB names another build of moe_oracle.c to load instead (the mutation
        # test runs the pins against copies with planted mistakes)
        path = os.environ.get("MOE_ORACLE_LIB") or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, u8, u16, f32 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint8,
                                  ctypes.c_uint16, ctypes.c_float)
        sig = {
            "oracle_bf16_to_f32": (f32, [u16]),
            "oracle_f32_to_bf16": (u16, [f32]),
            "oracle_e4m3_from_f32": (u8, [f32]),
            "oracle_e4m3_to_f32": (f32, [u8]),
            "oracle_e5m2_from_f32": (u8, [f32]),
            "oracle_e5m2_to_f32": (f32, [u8]),
            "oracle_e2m1_from_f32": (u8, [f32]),
            "oracle_e2m1_to_f32": (f32, [u8]),
            "oracle_code_row_bytes": (i32, [i32, i32]),
            "oracle_int8_from_f32": (ctypes.c_int8, [f32]),
            "oracle_e8m0_from_scale": (u8, [f32]),
            "oracle_f32_to_f16": (u16, [f32]),
            "oracle_f16_to_f32": (f32, [u16]),
            "oracle_int8_from_f16": (ctypes.c_int8, [u16]),
            "oracle_combine_block_count": (i32, [i32]),
            "oracle_combine_quant_row": (None, [P, i32, P, P]),
            "oracle_combine_quant_row_tok": (None, [i32, P, i32, P, P]),
            "oracle_combine_dequant_row": (None, [P, P, i32, P]),
            "oracle_combine_quantize": (i32, [P] * 5),
            "oracle_combine_int8": (i32, [P] * 13),
            "oracle_combine_int8_token": (i32, [P] * 10 + [i32, i32, P, P, P]),
            "oracle_expand_scales": (i32, [P] * 5),
            "oracle_combine_scatter": (i32, [P] * 12),
            "oracle_mx_scale_count": (i32, [i32]),
            "oracle_code_type": (i32, [i32, i32]),
            "oracle_scale_count": (i32, [i32, i32]),
            "oracle_quant_row": (i32, [i32, i32, P, P, i32, i32, P, P]),
            "oracle_quant_row_tok": (i32, [i32, i32, i32, P, P, i32, i32, P, P]),
            "oracle_quant_int8_row": (None, [P, P, i32, P, P]),
            "oracle_quant_mx_row": (None, [P, i32, i32, P, P]),
            "oracle_route": (i32, [P, P, P, P, P]),
            "oracle_recv_counts": (i32, [P, P, P, P, P]),
            "oracle_dest_row": (i64, [P, P, P, i32, i32, i32]),
            "oracle_dispatch": (i32, [P] * 13),
            "oracle_combine_token": (i32, [P] * 9 + [i32, i32, P, P]),
            "oracle_combine": (i32, [P] * 11),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous array of the given dtype, or None."""
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def make_cfg(W, E, BS, H, K, quant_mode=0, zero_expert_num=0, copy_expert_num=0,
             expert_token_nums_type=1, mask_kind=0, out_dtype=0, scales_kind=0,
             scale_format=0, token_dtype=TOKEN_BF16):
    return OracleCfg(W, E, BS, H, K, quant_mode, zero_expert_num, copy_expert_num,
                     expert_token_nums_type, mask_kind, out_dtype, scales_kind, scale_format,
                     token_dtype)


def _ref(cfg):
    return ctypes.byref(cfg)


# -- scalar helpers ------------------------------------------------------------------------

def bf16_to_f32(b):
    return _load().oracle_bf16_to_f32(int(b))


def f32_to_bf16(f):
    return _load().oracle_f32_to_bf16(float(f))


def e4m3_from_f32(v):
    return _load().oracle_e4m3_from_f32(float(v))


def e4m3_to_f32(code):
    return _load().oracle_e4m3_to_f32(int(code))


def e5m2_from_f32(v):
    return _load().oracle_e5m2_from_f32(float(v))


def e5m2_to_f32(code):
    return _load().oracle_e5m2_to_f32(int(code))


def e2m1_from_f32(v):
    return _load().oracle_e2m1_from_f32(float(v))


def e2m1_to_f32(code):
    return _load().oracle_e2m1_to_f32(int(code))


def code_row_bytes(ct, H):
    return _load().oracle_code_row_bytes(int(ct), int(H))


def int8_from_f32(v):
    return _load().oracle_int8_from_f32(float(v))


def e8m0_from_scale(s):
    return _load().oracle_e8m0_from_scale(float(s))


def f32_to_f16(f):
    return _load().oracle_f32_to_f16(float(f))


def f16_to_f32(h):
    return _load().oracle_f16_to_f32(int(h))


def int8_from_f16(h):
    return _load().oracle_int8_from_f16(int(h))


def combine_block_count(H):
    return _load().oracle_combine_block_count(int(H))


def mx_scale_count(H):
    return _load().oracle_mx_scale_count(int(H))


def code_type(quant_mode, out_dtype=0):
    return _load().oracle_code_type(int(quant_mode), int(out_dtype))


def scale_count(quant_mode, H):
    return _load().oracle_scale_count(int(quant_mode), int(H))


def code_np_dtype(ct):
    return {CODE_BF16: np.uint16, CODE_INT8: np.int8}.get(ct, np.uint8)


# -- rows ----------------------------------------------------------------------------------

def quant_int8_row(x_bf16, smooth=None):
    x = _c(x_bf16, np.uint16)
    sm = _c(smooth, np.float32)
    H = x.shape[0]
    q = np.empty(H, np.int8)
    sc = np.empty(1, np.float32)
    _load().oracle_quant_int8_row(_p(x), _p(sm), H, _p(q), _p(sc))
    return q, sc[0]


def quant_mx_row(x_bf16, clip):
    x = _c(x_bf16, np.uint16)
    H = x.shape[0]
    codes = np.empty(H, np.uint8)
    scales = np.empty(mx_scale_count(H), np.float32)
    _load().oracle_quant_mx_row(_p(x), H, 1 if clip else 0, _p(codes), _p(scales))
    return codes, scales


def quant_row(quant_mode, x_bf16, pre=None, out_dtype=0, token_dtype=TOKEN_BF16):
    """Quantize one row (bf16 bit patterns, or binary16 with token_dtype=TOKEN_F16); pre is
    None, a 1-element array (scalar) or an H-element row.  Returns (codes, scales) with codes
    int8 for the int8 type, else uint8."""
    x = _c(x_bf16, np.uint16)
    H = x.shape[0]
    ct = code_type(quant_mode, out_dtype)
    pr = _c(pre, np.float32)
    codes = np.empty(code_row_bytes(ct, H) // np.dtype(code_np_dtype(ct)).itemsize,
                     code_np_dtype(ct))
    scales = np.empty(max(1, scale_count(quant_mode, H)), np.float32)
    rc = _load().oracle_quant_row_tok(int(token_dtype), int(quant_mode), ct, _p(x), _p(pr),
                                      0 if pr is None else pr.shape[0], H, _p(codes),
                                      _p(scales))
    if rc != 0:
        raise ValueError(f"oracle_quant_row rejected the arguments (rc={rc})")
    return codes, scales[:scale_count(quant_mode, H)]


# -- routing -------------------------------------------------------------------------------

def route(cfg, expert_ids, mask=None):
    ids = _c(expert_ids, np.int32)
    m = _c(mask, np.uint8)
    cnt = np.empty((cfg.W, cfg.E), np.int32)
    eidx = np.empty((cfg.W, cfg.BS, cfg.K), np.int32)
    rc = _load().oracle_route(_ref(cfg), _p(ids), _p(m), _p(cnt), _p(eidx))
    if rc != 0:
        raise ValueError(f"oracle_route rejected the input (rc={rc})")
    return cnt, eidx


def recv_counts(cfg, cnt):
    L = cfg.E // cfg.W
    cnt = _c(cnt, np.int32)
    erc = np.empty((cfg.W, L * cfg.W), np.int32)
    etn = np.empty((cfg.W, L), np.int64)
    off = np.empty(cfg.W + 1, np.int64)
    _load().oracle_recv_counts(_ref(cfg), _p(cnt), _p(erc), _p(etn), _p(off))
    return erc, etn, off


def dest_row(cfg, ep_recv_count, recv_offsets, s, e, ordinal):
    erc = _c(ep_recv_count, np.int32)
    off = _c(recv_offsets, np.int64)
    return _load().oracle_dest_row(_ref(cfg), _p(erc), _p(off), int(s), int(e), int(ordinal))


def dispatch(cfg, x, expert_ids, scales=None, mask=None, cap=None):
    """Whole dispatch.  `scales` is the quantization scales tensor of cfg.scales_kind (a
    1-element array, an [H] row or an [E][H] table).  Returns a dict of numpy arrays; rows of
    expand_x / dynamic_scales / assist_info past recv_offsets[W] are left zero."""
    W, BS, H, K, L = cfg.W, cfg.BS, cfg.H, cfg.K, cfg.E // cfg.W
    x = _c(x, np.uint16)
    ids = _c(expert_ids, np.int32)
    sm = _c(scales, np.float32)
    m = _c(mask, np.uint8)
    cap = W * BS * K if cap is None else cap
    ct = code_type(cfg.quant_mode, cfg.out_dtype)
    if ct < 0:
        raise ValueError("quant_mode and out_dtype do not go together")
    ns = scale_count(cfg.quant_mode, H)
    ex = np.zeros((cap, code_row_bytes(ct, H) // np.dtype(code_np_dtype(ct)).itemsize),
                  code_np_dtype(ct))
    sdt = np.uint8 if cfg.scale_format == 1 else np.float32
    ds = np.zeros(1, sdt) if ns == 0 else np.zeros((cap,) if ns == 1 else (cap, ns), sdt)
    eidx = np.empty((W, BS, K), np.int32)
    ai = np.zeros((cap, 3), np.int32)
    erc = np.empty((W, L * W), np.int32)
    etn = np.empty((W, L), np.int64)
    off = np.empty(W + 1, np.int64)
    cnt = np.empty((W, cfg.E), np.int32)
    rc = _load().oracle_dispatch(_ref(cfg), _p(x), _p(ids), _p(sm), _p(m), _p(ex), _p(ds),
                                 _p(eidx), _p(ai), _p(erc), _p(etn), _p(off), _p(cnt))
    if rc != 0:
        raise ValueError(f"oracle_dispatch rejected the input (rc={rc})")
    out = dict(expand_x=ex, expand_idx=eidx, assist_info=ai, ep_recv_count=erc,
               expert_token_nums=etn, recv_offsets=off, cnt=cnt)
    if ns != 0:
        out["dynamic_scales"] = ds
    return out


def combine(cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
            recv_offsets, mask=None, ori_x=None):
    eo = _c(expert_out, np.uint16)
    ids = _c(expert_ids, np.int32)
    eidx = _c(expand_idx, np.int32)
    w = _c(expert_scales, np.float32)
    erc = _c(ep_recv_count, np.int32)
    off = _c(recv_offsets, np.int64)
    m = _c(mask, np.uint8)
    ox = _c(ori_x, np.uint16)
    y = np.empty((cfg.W, cfg.BS, cfg.H), np.uint16)
    acc = np.empty(cfg.H, np.float32)
    rc = _load().oracle_combine(_ref(cfg), _p(eo), _p(ids), _p(eidx), _p(w), _p(erc),
                                _p(off), _p(m), _p(ox), _p(y), _p(acc))
    if rc != 0:
        raise ValueError(f"oracle_combine rejected the input (rc={rc})")
    return y


def combine_token(cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
                  recv_offsets, s, i, mask=None, ori_x=None):
    """Combine for one source token (s, i); the big arrays are passed without copying when
    they are already contiguous in the right dtype."""
    eo = _c(expert_out, np.uint16)
    ids = _c(expert_ids, np.int32)
    eidx = _c(expand_idx, np.int32)
    w = _c(expert_scales, np.float32)
    erc = _c(ep_recv_count, np.int32)
    off = _c(recv_offsets, np.int64)
    m = _c(mask, np.uint8)
    ox = _c(ori_x, np.uint16)
    y = np.empty(cfg.H, np.uint16)
    acc = np.empty(cfg.H, np.float32)
    rc = _load().oracle_combine_token(_ref(cfg), _p(eo), _p(ids), _p(eidx), _p(w), _p(erc),
                                      _p(off), _p(m), _p(ox), int(s), int(i), _p(acc), _p(y))
    if rc != 0:
        raise ValueError(f"oracle_combine_token rejected the input (rc={rc})")
    return y


# -- combine-side int8 block quantization ------------------------------------------------------

def combine_quant_row(row_bf16, token_dtype=TOKEN_BF16):
    x = _c(row_bf16, np.uint16)
    H = x.shape[0]
    q = np.empty(H, np.int8)
    sc = np.empty(combine_block_count(H), np.float32)
    _load().oracle_combine_quant_row_tok(int(token_dtype), _p(x), H, _p(q), _p(sc))
    return q, sc


def combine_dequant_row(q, scales):
    q = _c(q, np.int8)
    sc = _c(scales, np.float32)
    out = np.empty(q.shape[0], np.float32)
    _load().oracle_combine_dequant_row(_p(q), _p(sc), q.shape[0], _p(out))
    return out


def combine_quantize(cfg, expert_out, recv_offsets):
    """Codes [cap][H] int8 and scales [cap][Ceil(H,8)] fp32 of the rows [0, recv_offsets[W]);
    later rows are left zero."""
    eo = _c(expert_out, np.uint16)
    off = _c(recv_offsets, np.int64)
    cap = eo.shape[0]
    codes = np.zeros((cap, cfg.H), np.int8)
    scales = np.zeros((cap, combine_block_count(cfg.H)), np.float32)
    _load().oracle_combine_quantize(_ref(cfg), _p(eo), _p(off), _p(codes), _p(scales))
    return codes, scales


def combine_int8(cfg, codes, scales, expert_ids, expand_idx, expert_scales, ep_recv_count,
                 recv_offsets, mask=None, ori_x=None):
    q = _c(codes, np.int8)
    sc = _c(scales, np.float32)
    ids = _c(expert_ids, np.int32)
    eidx = _c(expand_idx, np.int32)
    w = _c(expert_scales, np.float32)
    erc = _c(ep_recv_count, np.int32)
    off = _c(recv_offsets, np.int64)
    m = _c(mask, np.uint8)
    ox = _c(ori_x, np.uint16)
    y = np.empty((cfg.W, cfg.BS, cfg.H), np.uint16)
    acc = np.empty(cfg.H, np.float32)
    row = np.empty(cfg.H, np.float32)
    rc = _load().oracle_combine_int8(_ref(cfg), _p(q), _p(sc), _p(ids), _p(eidx), _p(w),
                                     _p(erc), _p(off), _p(m), _p(ox), _p(y), _p(acc), _p(row))
    if rc != 0:
        raise ValueError(f"oracle_combine_int8 rejected the input (rc={rc})")
    return y


# -- weights with the rows, scatter-back combine ---------------------------------------------

def expand_scales(cfg, assist_info, recv_offsets, expert_scales, cap):
    ai = _c(assist_info, np.int32)
    off = _c(recv_offsets, np.int64)
    w = _c(expert_scales, np.float32)
    out = np.zeros(cap, np.float32)
    rc = _load().oracle_expand_scales(_ref(cfg), _p(ai), _p(off), _p(w), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_expand_scales rejected the input (rc={rc})")
    return out


def combine_scatter(cfg, expert_out, assist_info, recv_offsets, expert_ids, expert_scales,
                    mask=None, ori_x=None, shared_x=None):
    eo = _c(expert_out, np.uint16)
    ai = _c(assist_info, np.int32)
    off = _c(recv_offsets, np.int64)
    ids = _c(expert_ids, np.int32)
    w = _c(expert_scales, np.float32)
    m = _c(mask, np.uint8)
    ox = _c(ori_x, np.uint16)
    sx = _c(shared_x, np.uint16)
    y = np.empty((cfg.W, cfg.BS, cfg.H), np.uint16)
    window = np.empty(cfg.W * cfg.BS * cfg.K * cfg.H, np.uint16)
    acc = np.empty(cfg.H, np.float32)
    rc = _load().oracle_combine_scatter(_ref(cfg), _p(eo), _p(ai), _p(off), _p(ids), _p(w),
                                        _p(m), _p(ox), _p(sx), _p(y), _p(window), _p(acc))
    if rc != 0:
        raise ValueError(f"oracle_combine_scatter rejected the input (rc={rc})")
    return y


def combine_int8_token(cfg, codes, scales, expert_ids, expand_idx, expert_scales,
                       ep_recv_count, recv_offsets, s, i, mask=None, ori_x=None):
    """The int8 combine for one source token (s, i)."""
    q = _c(codes, np.int8)
    sc = _c(scales, np.float32)
    ids = _c(expert_ids, np.int32)
    eidx = _c(expand_idx, np.int32)
    w = _c(expert_scales, np.float32)
    erc = _c(ep_recv_count, np.int32)
    off = _c(recv_offsets, np.int64)
    m = _c(mask, np.uint8)
    ox = _c(ori_x, np.uint16)
    y = np.empty(cfg.H, np.uint16)
    acc = np.empty(cfg.H, np.float32)
    row = np.empty(cfg.H, np.float32)
    rc = _load().oracle_combine_int8_token(_ref(cfg), _p(q), _p(sc), _p(ids), _p(eidx), _p(w),
                                           _p(erc), _p(off), _p(m), _p(ox), int(s), int(i),
                                           _p(acc), _p(row), _p(y))
    if rc != 0:
        raise ValueError(f"oracle_combine_int8_token rejected the input (rc={rc})")
    return y
