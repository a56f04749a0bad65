"""ctypes binding of libmoe_dc.so: argument marshalling only.

Function names mirror the C ABI in include/moe_dc.h.  Every step of dispatch and combine runs
in the library's HIP kernels; this module checks tensor dtypes/shapes/devices, passes raw
device pointers and the current HIP stream (with the tensors' device current, which the
library launches on), and turns a negative status into an exception.
It never falls back to another implementation: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = 0, -1, -2, -3, -4
MOE_DTYPE_DEFAULT, MOE_DTYPE_INT8, MOE_DTYPE_E4M3, MOE_DTYPE_E5M2, MOE_DTYPE_E2M1 = 0, 1, 2, 3, 4
MOE_SCALES_NONE, MOE_SCALES_SCALAR, MOE_SCALES_SHARED, MOE_SCALES_PER_EXPERT = 0, 1, 2, 3
MOE_SCALE_FP32, MOE_SCALE_E8M0, MOE_SCALE_FP32_RECIPROCAL = 0, 1, 2
MOE_DC_FLAG_SEPARATE_ROUTE, MOE_DC_FLAG_CHECK_IDS = 1, 2
MOE_TOKEN_BF16, MOE_TOKEN_F16 = 0, 1
_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
           -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_DEVICE"}

EXPORTS = ("moe_dc_validate", "moe_dc_scales_per_row", "moe_dc_dispatch_workspace_bytes",
           "moe_dc_combine_scatter_workspace_bytes", "moe_dispatch",
           "moe_dispatch_no_workspace", "moe_combine",
           "moe_combine_scatter", "moe_combine_quantize", "moe_combine_int8",
           "moe_dc_last_error", "moe_dc_version")


class MoeDcConfig(ctypes.Structure):
    """Mirror of moe_dc_config."""
    _fields_ = [
        ("ep_world_size", ctypes.c_int32),
        ("moe_expert_num", ctypes.c_int32),
        ("bs", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("quant_mode", ctypes.c_int32),
        ("zero_expert_num", ctypes.c_int32),
        ("copy_expert_num", ctypes.c_int32),
        ("const_expert_num", ctypes.c_int32),
        ("expert_token_nums_type", ctypes.c_int32),
        ("mask_kind", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scales_kind", ctypes.c_int32),
        ("scale_format", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("token_dtype", ctypes.c_int32),
        ("expand_rows_capacity", ctypes.c_int64),
    ]

    @property
    def W(self):
        return self.ep_world_size

    @property
    def E(self):
        return self.moe_expert_num

    @property
    def L(self):
        return self.moe_expert_num // self.ep_world_size


class MoeDcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB) -> ctypes.CDLL:
    """Load libmoe_dc.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with combine_quant_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, cfgp = ctypes.c_void_p, ctypes.POINTER(MoeDcConfig)
    lib.moe_dc_validate.restype = ctypes.c_int
    lib.moe_dc_validate.argtypes = [cfgp]
    lib.moe_dc_scales_per_row.restype = ctypes.c_int32
    lib.moe_dc_scales_per_row.argtypes = [cfgp]
    lib.moe_dc_dispatch_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_dc_dispatch_workspace_bytes.argtypes = [cfgp]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [cfgp] + [P] * 13 + [P, ctypes.c_size_t, P]
    lib.moe_dispatch_no_workspace.restype = ctypes.c_int
    lib.moe_dispatch_no_workspace.argtypes = [cfgp] + [P] * 13 + [P]
    lib.moe_dc_combine_scatter_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_dc_combine_scatter_workspace_bytes.argtypes = [cfgp]
    lib.moe_combine_scatter.restype = ctypes.c_int
    lib.moe_combine_scatter.argtypes = [cfgp] + [P] * 9 + [P, ctypes.c_size_t, P]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [cfgp] + [P] * 9 + [P]
    lib.moe_combine_quantize.restype = ctypes.c_int
    lib.moe_combine_quantize.argtypes = [cfgp] + [P] * 4 + [P]
    lib.moe_combine_int8.restype = ctypes.c_int
    lib.moe_combine_int8.argtypes = [cfgp] + [P] * 10 + [P]
    lib.moe_dc_last_error.restype = ctypes.c_char_p
    lib.moe_dc_last_error.argtypes = []
    lib.moe_dc_version.restype = ctypes.c_char_p
    lib.moe_dc_version.argtypes = []
    _lib = lib
    return lib


def make_config(W, E, BS, H, K, quant_mode=0, zero_expert_num=0, copy_expert_num=0,
                const_expert_num=0, expert_token_nums_type=1, mask_kind=0, cap=None,
                out_dtype=MOE_DTYPE_DEFAULT, scales_kind=MOE_SCALES_NONE,
                scale_format=MOE_SCALE_FP32, flags=0, token_dtype=MOE_TOKEN_BF16):
    cap = W * BS * K if cap is None else cap
    return MoeDcConfig(W, E, BS, H, K, quant_mode, zero_expert_num, copy_expert_num,
                       const_expert_num, expert_token_nums_type, mask_kind, out_dtype,
                       scales_kind, scale_format, flags, token_dtype, cap)


def token_torch_dtype(cfg):
    """torch dtype of the token tensors (x, ori_x, shared_x, expert_out, y, mode-0
    expand_x): bfloat16, or float16 when cfg.token_dtype is MOE_TOKEN_F16."""
    return torch.float16 if cfg.token_dtype == MOE_TOKEN_F16 else torch.bfloat16


def code_type(cfg):
    """Element type of expand_x: 0 bf16, 1 int8, 2 E4M3, 3 E5M2 (the moe_dtype values)."""
    if cfg.quant_mode == 0:
        return 0
    if cfg.out_dtype != MOE_DTYPE_DEFAULT:
        return cfg.out_dtype
    return MOE_DTYPE_INT8 if cfg.quant_mode in (1, 2) else MOE_DTYPE_E4M3


def _check(status: int):
    if status != MOE_OK:
        raise MoeDcError(status, load_library().moe_dc_last_error().decode())


def moe_dc_last_error() -> str:
    return load_library().moe_dc_last_error().decode()


def moe_dc_version() -> str:
    return load_library().moe_dc_version().decode()


def moe_dc_validate(cfg: MoeDcConfig) -> int:
    return load_library().moe_dc_validate(ctypes.byref(cfg))


def moe_dc_scales_per_row(cfg: MoeDcConfig) -> int:
    return load_library().moe_dc_scales_per_row(ctypes.byref(cfg))


def moe_dc_dispatch_workspace_bytes(cfg: MoeDcConfig) -> int:
    return load_library().moe_dc_dispatch_workspace_bytes(ctypes.byref(cfg))


def _ptr(t, dtype=None, shape=None, name="tensor", device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_CODE_DTYPES = {0: torch.bfloat16, 1: torch.int8, 2: (torch.uint8, torch.float8_e4m3fn),
                3: (torch.uint8, torch.float8_e5m2), 4: torch.uint8}
_ALLOC_DTYPES = {0: torch.bfloat16, 1: torch.int8, 2: torch.uint8, 3: torch.uint8,
                 4: torch.uint8}


def code_row_elems(cfg):
    """Elements of one expand_x row in its tensor dtype: H, or H / 2 bytes for E2M1."""
    return cfg.hidden // 2 if code_type(cfg) == MOE_DTYPE_E2M1 else cfg.hidden


def _scales_shape(cfg):
    return {MOE_SCALES_SCALAR: (1,), MOE_SCALES_SHARED: (cfg.hidden,),
            MOE_SCALES_PER_EXPERT: (cfg.moe_expert_num, cfg.hidden)}.get(cfg.scales_kind)


def _dyn_scales_spec(cfg):
    """(dtype, shape) of dynamic_scales, or None when the mode has no scales."""
    ns = moe_dc_scales_per_row(cfg)
    if ns <= 0:
        return None
    cap = cfg.expand_rows_capacity
    dt = torch.uint8 if cfg.scale_format == MOE_SCALE_E8M0 else torch.float32
    return dt, ((cap,) if ns == 1 else (cap, ns))


class Launch:
    """One C-ABI call whose arguments were checked and marshalled once.  Calling it enqueues
    the same call again on `stream` (default: the current stream of its device), which costs
    only the foreign call: a plan for serving loops.  It keeps the tensors it was built from
    alive; write new inputs into them in place between calls (or capture calls in a graph)."""

    __slots__ = ("_fn", "_args", "_dev", "_index", "_keep")

    def __init__(self, fn, args, dev, keep):
        self._fn, self._args, self._dev, self._keep = fn, args, dev, keep
        self._index = dev.index if dev.index is not None else torch.cuda.current_device()

    def __call__(self, stream=None):
        if torch.cuda.current_device() != self._index:
            _launch(self._fn, self._args, self._dev, stream)
            return
        s = torch.cuda.current_stream(self._dev) if stream is None else stream
        status = self._fn(*self._args, ctypes.c_void_p(s.cuda_stream))
        if status != MOE_OK:
            _check(status)


def _launch(fn, args, dev, stream):
    with torch.cuda.device(dev):
        _check(fn(*args, _stream(dev, stream)))


def _dispatch_call(cfg, x, expert_ids, scales, x_active_mask, expand_x, dynamic_scales,
                   expand_idx, assist_info, ep_recv_count, expert_token_nums, recv_offsets,
                   workspace, expert_scales=None, expand_scales=None):
    W, BS, H, K, L, cap = (cfg.ep_world_size, cfg.bs, cfg.hidden, cfg.topk, cfg.L,
                           cfg.expand_rows_capacity)
    dev = x.device
    spec = _dyn_scales_spec(cfg)
    mshape = {1: (W, BS), 2: (W, BS, K)}.get(cfg.mask_kind)
    args = [
        _ptr(x, token_torch_dtype(cfg), (W, BS, H), "x", dev),
        _ptr(expert_ids, torch.int32, (W, BS, K), "expert_ids", dev),
        _ptr(scales, torch.float32, _scales_shape(cfg), "scales", dev),
        _ptr(x_active_mask, (torch.uint8, torch.bool), mshape, "x_active_mask", dev),
        _ptr(expert_scales, torch.float32, (W, BS, K), "expert_scales", dev),
        _ptr(expand_x, (token_torch_dtype(cfg) if code_type(cfg) == 0
                        else _CODE_DTYPES.get(code_type(cfg))), (cap, code_row_elems(cfg)), "expand_x",
             dev),
        _ptr(dynamic_scales, None if spec is None else spec[0],
             None if spec is None else spec[1], "dynamic_scales", dev),
        _ptr(expand_idx, torch.int32, (W, BS, K), "expand_idx", dev),
        _ptr(assist_info, torch.int32, (cap, 3), "assist_info", dev),
        _ptr(ep_recv_count, torch.int32, (W, L * W), "ep_recv_count", dev),
        _ptr(expert_token_nums, torch.int64, (W, L), "expert_token_nums", dev),
        _ptr(recv_offsets, torch.int64, (W + 1,), "recv_offsets", dev),
        _ptr(expand_scales, torch.float32, (cap,), "expand_scales", dev),
        _ptr(workspace, torch.uint8, None, "workspace", dev),
    ]
    ws_bytes = 0 if workspace is None else workspace.numel()
    return (load_library().moe_dispatch,
            (ctypes.byref(cfg), *args, ctypes.c_size_t(ws_bytes)), dev)


def moe_dispatch(cfg, x, expert_ids, scales, x_active_mask, expand_x, dynamic_scales,
                 expand_idx, assist_info, ep_recv_count, expert_token_nums, recv_offsets,
                 workspace, stream=None, expert_scales=None, expand_scales=None):
    """Enqueue one dispatch on `stream` (default: the current stream of x's device).
    `scales` is the quantization scales tensor of cfg.scales_kind ([1], [H] or [E][H]);
    expert_scales [W][BS][K] and expand_scales [cap] (the rows' weights) go together."""
    _launch(*_dispatch_call(cfg, x, expert_ids, scales, x_active_mask, expand_x,
                            dynamic_scales, expand_idx, assist_info, ep_recv_count,
                            expert_token_nums, recv_offsets, workspace, expert_scales,
                            expand_scales), stream)


def moe_dispatch_no_workspace(cfg, x, expert_ids, scales, x_active_mask, expand_x,
                              dynamic_scales, expand_idx, assist_info, ep_recv_count,
                              expert_token_nums, recv_offsets, stream=None, expert_scales=None,
                              expand_scales=None):
    """Enqueue one dispatch without a workspace (the library's own static scratch is used);
    the arguments are moe_dispatch's, less the workspace."""
    fn, args, dev = _dispatch_call(cfg, x, expert_ids, scales, x_active_mask, expand_x,
                                   dynamic_scales, expand_idx, assist_info, ep_recv_count,
                                   expert_token_nums, recv_offsets, None, expert_scales,
                                   expand_scales)
    # moe_dispatch's argument list without its last two (workspace, workspace_bytes)
    _launch(load_library().moe_dispatch_no_workspace, args[:-2], dev, stream)


def _combine_call(cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
                  recv_offsets, x_active_mask, ori_x, y):
    W, BS, H, K, L, cap = (cfg.ep_world_size, cfg.bs, cfg.hidden, cfg.topk, cfg.L,
                           cfg.expand_rows_capacity)
    dev = y.device
    mshape = {1: (W, BS), 2: (W, BS, K)}.get(cfg.mask_kind)
    args = [
        _ptr(expert_out, token_torch_dtype(cfg), (cap, H), "expert_out", dev),
        _ptr(expert_ids, torch.int32, (W, BS, K), "expert_ids", dev),
        _ptr(expand_idx, torch.int32, (W, BS, K), "expand_idx", dev),
        _ptr(expert_scales, torch.float32, (W, BS, K), "expert_scales", dev),
        _ptr(ep_recv_count, torch.int32, (W, L * W), "ep_recv_count", dev),
        _ptr(recv_offsets, torch.int64, (W + 1,), "recv_offsets", dev),
        _ptr(x_active_mask, (torch.uint8, torch.bool), mshape, "x_active_mask", dev),
        _ptr(ori_x, token_torch_dtype(cfg), (W, BS, H), "ori_x", dev),
        _ptr(y, token_torch_dtype(cfg), (W, BS, H), "y", dev),
    ]
    return load_library().moe_combine, (ctypes.byref(cfg), *args), dev


def moe_combine(cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
                recv_offsets, x_active_mask, ori_x, y, stream=None):
    """Enqueue one combine on `stream` (default: the current stream of y's device)."""
    _launch(*_combine_call(cfg, expert_out, expert_ids, expand_idx, expert_scales,
                           ep_recv_count, recv_offsets, x_active_mask, ori_x, y), stream)


def moe_dc_combine_scatter_workspace_bytes(cfg: MoeDcConfig) -> int:
    return load_library().moe_dc_combine_scatter_workspace_bytes(ctypes.byref(cfg))


def _combine_scatter_call(cfg, expert_out, assist_info, recv_offsets, expert_ids,
                          expert_scales, x_active_mask, ori_x, shared_x, y, workspace):
    W, BS, H, K, cap = (cfg.ep_world_size, cfg.bs, cfg.hidden, cfg.topk,
                        cfg.expand_rows_capacity)
    dev = y.device
    mshape = {1: (W, BS), 2: (W, BS, K)}.get(cfg.mask_kind)
    args = [
        _ptr(expert_out, token_torch_dtype(cfg), (cap, H), "expert_out", dev),
        _ptr(assist_info, torch.int32, (cap, 3), "assist_info", dev),
        _ptr(recv_offsets, torch.int64, (W + 1,), "recv_offsets", dev),
        _ptr(expert_ids, torch.int32, (W, BS, K), "expert_ids", dev),
        _ptr(expert_scales, torch.float32, (W, BS, K), "expert_scales", dev),
        _ptr(x_active_mask, (torch.uint8, torch.bool), mshape, "x_active_mask", dev),
        _ptr(ori_x, token_torch_dtype(cfg), (W, BS, H), "ori_x", dev),
        _ptr(shared_x, token_torch_dtype(cfg), (W, BS, H), "shared_x", dev),
        _ptr(y, token_torch_dtype(cfg), (W, BS, H), "y", dev),
        _ptr(workspace, torch.uint8, None, "workspace", dev),
    ]
    ws_bytes = 0 if workspace is None else workspace.numel()
    return (load_library().moe_combine_scatter,
            (ctypes.byref(cfg), *args, ctypes.c_size_t(ws_bytes)), dev)


def moe_combine_scatter(cfg, expert_out, assist_info, recv_offsets, expert_ids, expert_scales,
                        x_active_mask, ori_x, shared_x, y, workspace, stream=None):
    """Enqueue one scatter-back combine (rows return by their assist_info triples)."""
    _launch(*_combine_scatter_call(cfg, expert_out, assist_info, recv_offsets, expert_ids,
                                   expert_scales, x_active_mask, ori_x, shared_x, y,
                                   workspace), stream)


def combine_block_count(cfg):
    """fp32 block scales per row of the combine-side int8 quantization: Ceil(H, 8)."""
    return (cfg.hidden + 7) // 8


def _combine_quantize_call(cfg, expert_out, recv_offsets, codes, block_scales):
    W, H, cap = cfg.ep_world_size, cfg.hidden, cfg.expand_rows_capacity
    dev = codes.device
    args = [
        _ptr(expert_out, token_torch_dtype(cfg), (cap, H), "expert_out", dev),
        _ptr(recv_offsets, torch.int64, (W + 1,), "recv_offsets", dev),
        _ptr(codes, torch.int8, (cap, H), "codes", dev),
        _ptr(block_scales, torch.float32, (cap, combine_block_count(cfg)), "block_scales",
             dev),
    ]
    return load_library().moe_combine_quantize, (ctypes.byref(cfg), *args), dev


def moe_combine_quantize(cfg, expert_out, recv_offsets, codes, block_scales, stream=None):
    """Enqueue the expert-side int8 block quantization of rows [0, recv_offsets[W])."""
    _launch(*_combine_quantize_call(cfg, expert_out, recv_offsets, codes, block_scales), stream)


def _combine_int8_call(cfg, codes, block_scales, expert_ids, expand_idx, expert_scales,
                       ep_recv_count, recv_offsets, x_active_mask, ori_x, y):
    W, BS, H, K, L, cap = (cfg.ep_world_size, cfg.bs, cfg.hidden, cfg.topk, cfg.L,
                           cfg.expand_rows_capacity)
    dev = y.device
    mshape = {1: (W, BS), 2: (W, BS, K)}.get(cfg.mask_kind)
    args = [
        _ptr(codes, torch.int8, (cap, H), "codes", dev),
        _ptr(block_scales, torch.float32, (cap, combine_block_count(cfg)), "block_scales",
             dev),
        _ptr(expert_ids, torch.int32, (W, BS, K), "expert_ids", dev),
        _ptr(expand_idx, torch.int32, (W, BS, K), "expand_idx", dev),
        _ptr(expert_scales, torch.float32, (W, BS, K), "expert_scales", dev),
        _ptr(ep_recv_count, torch.int32, (W, L * W), "ep_recv_count", dev),
        _ptr(recv_offsets, torch.int64, (W + 1,), "recv_offsets", dev),
        _ptr(x_active_mask, (torch.uint8, torch.bool), mshape, "x_active_mask", dev),
        _ptr(ori_x, token_torch_dtype(cfg), (W, BS, H), "ori_x", dev),
        _ptr(y, token_torch_dtype(cfg), (W, BS, H), "y", dev),
    ]
    return load_library().moe_combine_int8, (ctypes.byref(cfg), *args), dev


def moe_combine_int8(cfg, codes, block_scales, expert_ids, expand_idx, expert_scales,
                     ep_recv_count, recv_offsets, x_active_mask, ori_x, y, stream=None):
    """Enqueue one combine over int8 block-quantized expert rows."""
    _launch(*_combine_int8_call(cfg, codes, block_scales, expert_ids, expand_idx, expert_scales,
                                ep_recv_count, recv_offsets, x_active_mask, ori_x, y), stream)


# -- allocation helpers (torch owns the memory; the library never allocates) ----------------

def alloc_dispatch_outputs(cfg, device="cuda"):
    """Empty output tensors and a workspace sized for cfg."""
    _check(moe_dc_validate(cfg))
    W, BS, H, K, L, cap = (cfg.ep_world_size, cfg.bs, cfg.hidden, cfg.topk, cfg.L,
                           cfg.expand_rows_capacity)
    spec = _dyn_scales_spec(cfg)
    return dict(
        expand_x=torch.empty((cap, code_row_elems(cfg)),
                             dtype=(token_torch_dtype(cfg) if code_type(cfg) == 0
                                    else _ALLOC_DTYPES[code_type(cfg)]),
                             device=device),
        dynamic_scales=(None if spec is None else
                        torch.empty(spec[1], dtype=spec[0], device=device)),
        expand_idx=torch.empty((W, BS, K), dtype=torch.int32, device=device),
        assist_info=torch.empty((cap, 3), dtype=torch.int32, device=device),
        ep_recv_count=torch.empty((W, L * W), dtype=torch.int32, device=device),
        expert_token_nums=torch.empty((W, L), dtype=torch.int64, device=device),
        recv_offsets=torch.empty((W + 1,), dtype=torch.int64, device=device),
        workspace=torch.empty((moe_dc_dispatch_workspace_bytes(cfg),), dtype=torch.uint8,
                              device=device),
    )


def _new_y(cfg, like):
    return torch.empty((cfg.ep_world_size, cfg.bs, cfg.hidden), dtype=token_torch_dtype(cfg),
                       device=like.device)


# Each prepare_* checks and marshals one call once and returns (launch, outputs): calling
# `launch(stream=None)` enqueues the same call again with the same tensors, costing only the
# foreign call.  The plain functions below prepare and launch once.

def prepare_dispatch(cfg, x, expert_ids, scales=None, x_active_mask=None, out=None,
                     expert_scales=None):
    """Plan for moe_dispatch: (launch, output dict; "expand_scales" when expert_scales is
    given).  Write new x / expert_ids / mask contents in place between launches."""
    o = alloc_dispatch_outputs(cfg, x.device) if out is None else out
    if expert_scales is not None and o.get("expand_scales") is None:
        o["expand_scales"] = torch.empty((cfg.expand_rows_capacity,), dtype=torch.float32,
                                         device=x.device)
    fn, args, dev = _dispatch_call(
        cfg, x, expert_ids, scales, x_active_mask, o["expand_x"], o["dynamic_scales"],
        o["expand_idx"], o["assist_info"], o["ep_recv_count"], o["expert_token_nums"],
        o["recv_offsets"], o["workspace"], expert_scales,
        o.get("expand_scales") if expert_scales is not None else None)
    keep = (cfg, x, expert_ids, scales, x_active_mask, expert_scales, dict(o))
    return Launch(fn, args, dev, keep), o


def dispatch(cfg, x, expert_ids, scales=None, x_active_mask=None, out=None, stream=None,
             expert_scales=None):
    """Allocate (or reuse `out`) and enqueue moe_dispatch; returns the output dict (with
    "expand_scales" when expert_scales is given)."""
    launch, o = prepare_dispatch(cfg, x, expert_ids, scales, x_active_mask, out, expert_scales)
    launch(stream)
    return o


def prepare_combine(cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
                    recv_offsets, x_active_mask=None, ori_x=None, y=None):
    """Plan for moe_combine: (launch, y)."""
    y = _new_y(cfg, expert_out) if y is None else y
    fn, args, dev = _combine_call(cfg, expert_out, expert_ids, expand_idx, expert_scales,
                                  ep_recv_count, recv_offsets, x_active_mask, ori_x, y)
    keep = (cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
            recv_offsets, x_active_mask, ori_x, y)
    return Launch(fn, args, dev, keep), y


def combine(cfg, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
            recv_offsets, x_active_mask=None, ori_x=None, y=None, stream=None):
    """Allocate (or reuse `y`) and enqueue moe_combine; returns y."""
    launch, y = prepare_combine(cfg, expert_out, expert_ids, expand_idx, expert_scales,
                                ep_recv_count, recv_offsets, x_active_mask, ori_x, y)
    launch(stream)
    return y


def prepare_combine_scatter(cfg, expert_out, assist_info, recv_offsets, expert_ids,
                            expert_scales, x_active_mask=None, ori_x=None, shared_x=None,
                            y=None, workspace=None):
    """Plan for moe_combine_scatter: (launch, y)."""
    dev = expert_out.device
    y = _new_y(cfg, expert_out) if y is None else y
    if workspace is None:
        workspace = torch.empty((moe_dc_combine_scatter_workspace_bytes(cfg),),
                                dtype=torch.uint8, device=dev)
    fn, args, d = _combine_scatter_call(cfg, expert_out, assist_info, recv_offsets,
                                        expert_ids, expert_scales, x_active_mask, ori_x,
                                        shared_x, y, workspace)
    keep = (cfg, expert_out, assist_info, recv_offsets, expert_ids, expert_scales,
            x_active_mask, ori_x, shared_x, y, workspace)
    return Launch(fn, args, d, keep), y


def combine_scatter(cfg, expert_out, assist_info, recv_offsets, expert_ids, expert_scales,
                    x_active_mask=None, ori_x=None, shared_x=None, y=None, workspace=None,
                    stream=None):
    """Allocate (or reuse `y` / `workspace`) and enqueue moe_combine_scatter; returns y."""
    launch, y = prepare_combine_scatter(cfg, expert_out, assist_info, recv_offsets,
                                        expert_ids, expert_scales, x_active_mask, ori_x,
                                        shared_x, y, workspace)
    launch(stream)
    return y


def prepare_combine_quantize(cfg, expert_out, recv_offsets, out=None):
    """Plan for moe_combine_quantize: (launch, (codes, block_scales))."""
    cap, H = cfg.expand_rows_capacity, cfg.hidden
    if out is None:
        out = (torch.empty((cap, H), dtype=torch.int8, device=expert_out.device),
               torch.empty((cap, combine_block_count(cfg)), dtype=torch.float32,
                           device=expert_out.device))
    fn, args, dev = _combine_quantize_call(cfg, expert_out, recv_offsets, out[0], out[1])
    return Launch(fn, args, dev, (cfg, expert_out, recv_offsets, out)), out


def combine_quantize(cfg, expert_out, recv_offsets, out=None, stream=None):
    """Allocate (or reuse `out` = (codes, block_scales)) and enqueue moe_combine_quantize."""
    launch, out = prepare_combine_quantize(cfg, expert_out, recv_offsets, out)
    launch(stream)
    return out


def prepare_combine_int8(cfg, codes, block_scales, expert_ids, expand_idx, expert_scales,
                         ep_recv_count, recv_offsets, x_active_mask=None, ori_x=None, y=None):
    """Plan for moe_combine_int8: (launch, y)."""
    y = _new_y(cfg, codes) if y is None else y
    fn, args, dev = _combine_int8_call(cfg, codes, block_scales, expert_ids, expand_idx,
                                       expert_scales, ep_recv_count, recv_offsets,
                                       x_active_mask, ori_x, y)
    keep = (cfg, codes, block_scales, expert_ids, expand_idx, expert_scales, ep_recv_count,
            recv_offsets, x_active_mask, ori_x, y)
    return Launch(fn, args, dev, keep), y


def combine_int8(cfg, codes, block_scales, expert_ids, expand_idx, expert_scales,
                 ep_recv_count, recv_offsets, x_active_mask=None, ori_x=None, y=None,
                 stream=None):
    """Allocate (or reuse `y`) and enqueue moe_combine_int8; returns y."""
    launch, y = prepare_combine_int8(cfg, codes, block_scales, expert_ids, expand_idx,
                                     expert_scales, ep_recv_count, recv_offsets,
                                     x_active_mask, ori_x, y)
    launch(stream)
    return y
