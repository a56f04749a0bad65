// api.cpp -- C ABI of libmoe_dc: host validation, workspace sizing and launch sequencing.
//
// Nothing here allocates device memory or synchronises the host; every launch goes to the
// caller's stream in order (route -> scan -> scatter for dispatch, or the scatter alone for a
// small batch, which routes in its own workgroups; index then gather for the scatter-back
// combine; one kernel for each of combine, combine quantize and int8 combine).
#include "moe_dc.h"
#include "dc_internal.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

moe_status ok()
{
    g_last_error.clear();
    return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Element type of expand_x for a quant mode and requested out_dtype, or -1 when the pair is
// not allowed ([LLD] 约束说明: mode 0 keeps the input type; mode 1 int8; mode 2 int8, E4M3
// or E5M2; mode 3 E4M3 or E5M2; modes 4/5 E4M3, E5M2 or E2M1).
int32_t resolve_code_type(int32_t mode, int32_t out_dtype)
{
    switch (mode) {
    case 0:
        return out_dtype == MOE_DTYPE_DEFAULT ? moe_dc::kCodeBf16 : -1;
    case 1:
        return out_dtype == MOE_DTYPE_DEFAULT || out_dtype == MOE_DTYPE_INT8 ? moe_dc::kCodeInt8
                                                                             : -1;
    case 2:
        if (out_dtype == MOE_DTYPE_DEFAULT || out_dtype == MOE_DTYPE_INT8) return moe_dc::kCodeInt8;
        if (out_dtype == MOE_DTYPE_E4M3) return moe_dc::kCodeE4m3;
        return out_dtype == MOE_DTYPE_E5M2 ? moe_dc::kCodeE5m2 : -1;
    default:
        if (out_dtype == MOE_DTYPE_DEFAULT || out_dtype == MOE_DTYPE_E4M3) return moe_dc::kCodeE4m3;
        if (out_dtype == MOE_DTYPE_E5M2) return moe_dc::kCodeE5m2;
        return out_dtype == MOE_DTYPE_E2M1 && mode >= 4 ? moe_dc::kCodeE2m1 : -1;
    }
}

// Range and divisibility rules of the ops-transformer article (约束说明; the wrapper's
// checks under 调用说明) and of low_latency_dispatch (约束说明).
moe_status check(const moe_dc_config* c, moe_dc::Shape* out)
{
    if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
    if ((c->flags & ~(MOE_DC_FLAG_SEPARATE_ROUTE | MOE_DC_FLAG_CHECK_IDS)) != 0)
        return fail(MOE_ERR_INVALID_ARG, "flags has unknown bits (0x%x)", c->flags);
    if (c->token_dtype != MOE_TOKEN_BF16 && c->token_dtype != MOE_TOKEN_F16)
        return fail(MOE_ERR_INVALID_ARG, "token_dtype %d is not one of 0 (bf16), 1 (fp16)",
                    c->token_dtype);
    if (c->ep_world_size < 2 || c->ep_world_size > 768)
        return fail(MOE_ERR_INVALID_ARG, "ep_world_size %d outside [2, 768]", c->ep_world_size);
    if (c->moe_expert_num <= 0 || c->moe_expert_num > 1024)
        return fail(MOE_ERR_INVALID_ARG, "moe_expert_num %d outside (0, 1024]", c->moe_expert_num);
    if (c->moe_expert_num % c->ep_world_size != 0)
        return fail(MOE_ERR_INVALID_ARG, "moe_expert_num %d is not a multiple of ep_world_size %d",
                    c->moe_expert_num, c->ep_world_size);
    const int32_t L = c->moe_expert_num / c->ep_world_size;
    if ((int64_t)L * c->ep_world_size > 2048)
        return fail(MOE_ERR_INVALID_ARG, "local_expert_num * ep_world_size exceeds 2048");
    if (c->bs < 1 || c->bs > 512) return fail(MOE_ERR_INVALID_ARG, "bs %d outside [1, 512]", c->bs);
    if (c->hidden < 1024 || c->hidden > 8192)
        return fail(MOE_ERR_INVALID_ARG, "hidden %d outside [1024, 8192]", c->hidden);
    if (c->zero_expert_num < 0 || c->copy_expert_num < 0 || c->const_expert_num < 0)
        return fail(MOE_ERR_INVALID_ARG, "special expert counts must be >= 0");
    const int64_t all_ids = (int64_t)c->moe_expert_num + c->zero_expert_num +
                            c->copy_expert_num + c->const_expert_num;
    if (all_ids >= INT32_MAX)
        return fail(MOE_ERR_INVALID_ARG, "expert id space reaches INT32_MAX");
    if (c->topk <= 0 || c->topk > 16)
        return fail(MOE_ERR_INVALID_ARG, "topk %d outside (0, 16]", c->topk);
    if (c->topk > all_ids)
        return fail(MOE_ERR_INVALID_ARG, "topk %d exceeds the number of experts", c->topk);
    if (c->const_expert_num != 0)
        return fail(MOE_ERR_UNSUPPORTED, "const experts are not supported");
    if (c->quant_mode < 0 || c->quant_mode > 5)
        return fail(MOE_ERR_INVALID_ARG, "quant_mode %d is not one of 0..5", c->quant_mode);
    const int32_t code_type = resolve_code_type(c->quant_mode, c->out_dtype);
    if (code_type < 0)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype %d is not allowed with quant_mode %d",
                    c->out_dtype, c->quant_mode);
    if (code_type == moe_dc::kCodeE2m1 && c->hidden % 2 != 0)
        return fail(MOE_ERR_INVALID_ARG, "E2M1 codes need an even hidden size");
    if (c->scales_kind < MOE_SCALES_NONE || c->scales_kind > MOE_SCALES_PER_EXPERT)
        return fail(MOE_ERR_INVALID_ARG, "scales_kind %d is not one of 0..3", c->scales_kind);
    if ((c->quant_mode == 0 || c->quant_mode >= 4) && c->scales_kind != MOE_SCALES_NONE)
        return fail(MOE_ERR_INVALID_ARG, "quant_mode %d takes no scales tensor", c->quant_mode);
    if (c->quant_mode == 1 && c->scales_kind == MOE_SCALES_NONE)
        return fail(MOE_ERR_INVALID_ARG, "quant_mode 1 needs a scales tensor");
    if (c->scale_format != MOE_SCALE_FP32 &&
        !((c->scale_format == MOE_SCALE_E8M0 || c->scale_format == MOE_SCALE_FP32_RECIPROCAL) &&
          c->quant_mode >= 4))
        return fail(MOE_ERR_INVALID_ARG, "scale_format %d is not allowed with quant_mode %d",
                    c->scale_format, c->quant_mode);
    if (c->expert_token_nums_type != 0 && c->expert_token_nums_type != 1)
        return fail(MOE_ERR_INVALID_ARG, "expert_token_nums_type must be 0 or 1");
    if (c->mask_kind < 0 || c->mask_kind > 2)
        return fail(MOE_ERR_INVALID_ARG, "mask_kind must be 0, 1 or 2");
    const int64_t need_rows = (int64_t)c->ep_world_size * c->bs * c->topk;
    if (c->expand_rows_capacity < need_rows)
        return fail(MOE_ERR_INVALID_ARG, "expand_rows_capacity %lld < W*BS*K = %lld",
                    (long long)c->expand_rows_capacity, (long long)need_rows);
    if (c->expand_rows_capacity >= ((int64_t)1 << 31))
        return fail(MOE_ERR_INVALID_ARG, "expand_rows_capacity must be below 2^31");
    if (out) {
        out->W = c->ep_world_size;
        out->E = c->moe_expert_num;
        out->L = L;
        out->BS = c->bs;
        out->H = c->hidden;
        out->K = c->topk;
        out->quant_mode = c->quant_mode;
        out->code_type = code_type;
        out->scales_kind = c->scales_kind;
        out->scale_format = c->scale_format;
        out->zero_end = c->moe_expert_num + c->zero_expert_num;
        out->id_end = out->zero_end + c->copy_expert_num;
        out->etn_type = c->expert_token_nums_type;
        out->mask_kind = c->mask_kind;
        const int32_t nb = (c->hidden + 31) / 32;
        out->scales_per_row = c->quant_mode <= 1   ? 0
                              : c->quant_mode == 2 ? 1
                              : c->quant_mode == 3 ? (c->hidden + 127) / 128
                                                   : nb + (nb & 1);
        out->cap = c->expand_rows_capacity;
        out->tok_f16 = c->token_dtype == MOE_TOKEN_F16 ? 1 : 0;
    }
    return MOE_OK;
}

}  // namespace

moe_status moe_dc::set_error(moe_status st, const char* msg)
{
    return fail(st, "%s", msg);
}

moe_status moe_dc::check_dispatch_args(const moe_dc_config* cfg, const void* x,
                                       const int32_t* expert_ids, const float* scales,
                                       const uint8_t* x_active_mask, const float* expert_scales,
                                       const void* expand_x, const void* dynamic_scales,
                                       const int32_t* expand_idx, const int32_t* assist_info,
                                       const int32_t* ep_recv_count,
                                       const int64_t* expert_token_nums,
                                       const int64_t* recv_offsets, const float* expand_scales,
                                       Shape* out)
{
    moe_dc::Shape sh;
    moe_status st = check(cfg, &sh);
    if (st != MOE_OK) return st;
    if (!x || !expert_ids || !expand_x || !expand_idx || !assist_info || !ep_recv_count ||
        !expert_token_nums || !recv_offsets)
        return fail(MOE_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if (sh.scales_per_row > 0 && !dynamic_scales)
        return fail(MOE_ERR_INVALID_ARG, "dynamic_scales is required for quant_mode %d",
                    sh.quant_mode);
    if ((sh.scales_kind != MOE_SCALES_NONE) != (scales != nullptr))
        return fail(MOE_ERR_INVALID_ARG,
                    "scales must be given iff scales_kind is not MOE_SCALES_NONE");
    if ((sh.mask_kind != 0) != (x_active_mask != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "x_active_mask must be given iff mask_kind != 0");
    if ((expert_scales != nullptr) != (expand_scales != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "expert_scales and expand_scales go together");
    if (out) *out = sh;
    return MOE_OK;
}

namespace {

moe_status device_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

moe_status moe_dc_validate(const moe_dc_config* cfg)
{
    moe_status st = check(cfg, nullptr);
    return st == MOE_OK ? ok() : st;
}

int32_t moe_dc_scales_per_row(const moe_dc_config* cfg)
{
    moe_dc::Shape sh;
    if (check(cfg, &sh) != MOE_OK) return -1;
    return sh.scales_per_row;
}

size_t moe_dc_dispatch_workspace_bytes(const moe_dc_config* cfg)
{
    moe_dc::Shape sh;
    if (check(cfg, &sh) != MOE_OK) return 0;
    return moe_dc::workspace_bytes(sh);
}

moe_status moe_dispatch(const moe_dc_config* cfg, const void* x, const int32_t* expert_ids,
                        const float* scales, const uint8_t* x_active_mask,
                        const float* expert_scales, void* expand_x, void* dynamic_scales,
                        int32_t* expand_idx, int32_t* assist_info, int32_t* ep_recv_count,
                        int64_t* expert_token_nums, int64_t* recv_offsets,
                        float* expand_scales, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    moe_dc::Shape sh;
    moe_status st = moe_dc::check_dispatch_args(cfg, x, expert_ids, scales, x_active_mask,
                                                expert_scales, expand_x, dynamic_scales,
                                                expand_idx, assist_info, ep_recv_count,
                                                expert_token_nums, recv_offsets,
                                                expand_scales, &sh);
    if (st != MOE_OK) return st;
    const size_t need = moe_dc::workspace_bytes(sh);
    if (!workspace || workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace_bytes);
    if (!aligned4(workspace))
        return fail(MOE_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* seg = reinterpret_cast<int32_t*>(ws + moe_dc::kWsSegOffset);
    const bool check_ids = (cfg->flags & MOE_DC_FLAG_CHECK_IDS) != 0;
    int32_t* bad_word = check_ids ? reinterpret_cast<int32_t*>(ws) : nullptr;
    int32_t* bad_counts =
        check_ids ? reinterpret_cast<int32_t*>(ws + moe_dc::ws_bad_counts_offset(sh)) : nullptr;
    const bool row_scales =
        sh.scales_kind == MOE_SCALES_SHARED || sh.scales_kind == MOE_SCALES_PER_EXPERT;
    const bool vec = sh.H % 8 == 0 && aligned16(x) && aligned16(expand_x) &&
                     (!row_scales || aligned16(scales));

    // A small batch routes inside the scatter launch (one launch instead of three).
    const bool fused = vec && (cfg->flags & MOE_DC_FLAG_SEPARATE_ROUTE) == 0 &&
                       moe_dc::fused_route_fits(sh);
    const moe_dc::FusedRoute fr{x_active_mask, ep_recv_count, expert_token_nums, recv_offsets,
                                bad_word, sh.id_end};
    if (!fused) {
        st = device_status(
            moe_dc::launch_route(sh, expert_ids, x_active_mask, expand_idx, seg, bad_counts, s),
            "route kernel launch");
        if (st != MOE_OK) return st;
        int32_t* totals = reinterpret_cast<int32_t*>(ws + moe_dc::ws_scan_totals_offset(sh));
        st = device_status(moe_dc::launch_scan(sh, seg, ep_recv_count, expert_token_nums,
                                               recv_offsets, bad_counts, bad_word, totals, s),
                           "scan kernel launch");
        if (st != MOE_OK) return st;
    }
    st = device_status(moe_dc::launch_scatter(sh, x, expert_ids, expand_idx, seg, scales,
                                              expert_scales, expand_x, dynamic_scales,
                                              assist_info, expand_scales, vec,
                                              fused ? &fr : nullptr, s),
                       "scatter kernel launch");
    if (st != MOE_OK) return st;
    return ok();
}

moe_status moe_combine(const moe_dc_config* cfg, const void* expert_out,
                       const int32_t* expert_ids, const int32_t* expand_idx,
                       const float* expert_scales, const int32_t* ep_recv_count,
                       const int64_t* recv_offsets, const uint8_t* x_active_mask,
                       const void* ori_x, void* y, void* stream)
{
    moe_dc::Shape sh;
    moe_status st = check(cfg, &sh);
    if (st != MOE_OK) return st;
    if (!expert_out || !expert_ids || !expand_idx || !expert_scales || !ep_recv_count ||
        !recv_offsets || !y)
        return fail(MOE_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if ((sh.mask_kind != 0) != (x_active_mask != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "x_active_mask must be given iff mask_kind != 0");
    if (cfg->copy_expert_num > 0 && !ori_x)
        return fail(MOE_ERR_INVALID_ARG, "ori_x is required when copy experts exist");
    const bool vec = sh.H % 8 == 0 && aligned16(expert_out) && aligned16(y) &&
                     (!ori_x || aligned16(ori_x));
    st = device_status(moe_dc::launch_combine(sh, expert_out, expert_ids, expand_idx,
                                              expert_scales, ep_recv_count, recv_offsets,
                                              x_active_mask, ori_x, y, vec,
                                              static_cast<hipStream_t>(stream)),
                       "combine kernel launch");
    if (st != MOE_OK) return st;
    return ok();
}

size_t moe_dc_combine_scatter_workspace_bytes(const moe_dc_config* cfg)
{
    moe_dc::Shape sh;
    if (check(cfg, &sh) != MOE_OK) return 0;
    return moe_dc::combine_scatter_workspace_bytes(sh);
}

moe_status moe_combine_scatter(const moe_dc_config* cfg, const void* expert_out,
                               const int32_t* assist_info, const int64_t* recv_offsets,
                               const int32_t* expert_ids, const float* expert_scales,
                               const uint8_t* x_active_mask, const void* ori_x,
                               const void* shared_x, void* y, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    moe_dc::Shape sh;
    moe_status st = check(cfg, &sh);
    if (st != MOE_OK) return st;
    if (!expert_out || !assist_info || !recv_offsets || !expert_ids || !expert_scales || !y)
        return fail(MOE_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if ((sh.mask_kind != 0) != (x_active_mask != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "x_active_mask must be given iff mask_kind != 0");
    if (cfg->copy_expert_num > 0 && !ori_x)
        return fail(MOE_ERR_INVALID_ARG, "ori_x is required when copy experts exist");
    const size_t need = moe_dc::combine_scatter_workspace_bytes(sh);
    if (!workspace || workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace_bytes);
    if (!aligned4(workspace))
        return fail(MOE_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    const bool vec = sh.H % 8 == 0 && aligned16(expert_out) && aligned16(y) &&
                     (!ori_x || aligned16(ori_x)) && (!shared_x || aligned16(shared_x));
    st = device_status(moe_dc::launch_combine_scatter(sh, expert_out, assist_info,
                                                      recv_offsets, expert_ids, expert_scales,
                                                      x_active_mask, ori_x, shared_x, y,
                                                      static_cast<int32_t*>(workspace), vec,
                                                      static_cast<hipStream_t>(stream)),
                       "scatter-back combine launch");
    if (st != MOE_OK) return st;
    return ok();
}

moe_status moe_combine_quantize(const moe_dc_config* cfg, const void* expert_out,
                                const int64_t* recv_offsets, int8_t* codes,
                                float* block_scales, void* stream)
{
    moe_dc::Shape sh;
    moe_status st = check(cfg, &sh);
    if (st != MOE_OK) return st;
    if (!expert_out || !recv_offsets || !codes || !block_scales)
        return fail(MOE_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    const bool vec = sh.H % 8 == 0 && aligned16(expert_out) && aligned8(codes);
    st = device_status(moe_dc::launch_combine_quantize(sh, expert_out, recv_offsets, codes,
                                                       block_scales, vec,
                                                       static_cast<hipStream_t>(stream)),
                       "combine quantize kernel launch");
    if (st != MOE_OK) return st;
    return ok();
}

moe_status moe_combine_int8(const moe_dc_config* cfg, const int8_t* codes,
                            const float* block_scales, const int32_t* expert_ids,
                            const int32_t* expand_idx, const float* expert_scales,
                            const int32_t* ep_recv_count, const int64_t* recv_offsets,
                            const uint8_t* x_active_mask, const void* ori_x, void* y,
                            void* stream)
{
    moe_dc::Shape sh;
    moe_status st = check(cfg, &sh);
    if (st != MOE_OK) return st;
    if (!codes || !block_scales || !expert_ids || !expand_idx || !expert_scales ||
        !ep_recv_count || !recv_offsets || !y)
        return fail(MOE_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if ((sh.mask_kind != 0) != (x_active_mask != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "x_active_mask must be given iff mask_kind != 0");
    if (cfg->copy_expert_num > 0 && !ori_x)
        return fail(MOE_ERR_INVALID_ARG, "ori_x is required when copy experts exist");
    const bool vec = sh.H % 8 == 0 && aligned8(codes) && aligned16(y) &&
                     (!ori_x || aligned16(ori_x));
    st = device_status(moe_dc::launch_combine_int8(sh, codes, block_scales, expert_ids,
                                                   expand_idx, expert_scales, ep_recv_count,
                                                   recv_offsets, x_active_mask, ori_x, y, vec,
                                                   static_cast<hipStream_t>(stream)),
                       "int8 combine kernel launch");
    if (st != MOE_OK) return st;
    return ok();
}

const char* moe_dc_last_error(void) { return g_last_error.c_str(); }

const char* moe_dc_version(void) { return "moe_dc 0.4.0 (gfx950)"; }

}  // extern "C"
