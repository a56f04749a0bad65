/*
 * moe_dc.h -- MoE Dispatch/Combine for one AMD Instinct MI355X (gfx950), C ABI.
 *
 * The library implements the data path of the MoE dispatch and combine operators described
 * by these pages (cited below by the tags in brackets):
 *   [DDD] "MoeDistributeDispatch和MoeDistributeCombine算子设计介绍" (gitcode design doc)
 *   [LLD] "low_latency_dispatch" (hiascend API doc): 计算公式, 约束说明
 *   [OPS] "CANN ops-transformer 算子解析：MoeDistributeDispatchV3 的 EP 域 Token 分发与动态量化
 *         通信实现" (mwwr.cn): 功能说明, 参数说明, 约束说明, 调用说明, 接口级量化模式扩展
 *   [SMP] "CANN MoE Dispatch/Combine 通信算子性能优化实践：Kernel 直调与 ACL SHMEM 实现专家分发
 *         与聚合" (lqnn.cn): Dispatch 功能介绍, Combine 功能介绍, 通信前量化
 *
 * All W logical expert-parallel (EP) ranks live in the HBM of one GPU.  The pages' all-to-all
 * exchange therefore becomes a device-local permutation: dispatch writes every routed pick
 * straight to its final row of the receivers' packed buffer, and combine gathers from there.
 *
 * Notation: W ranks, E routed experts (L = E / W per rank, rank r owns [r*L, (r+1)*L)),
 * BS tokens per source rank, H hidden size, K picks per token.  A "pick" is (s, i, k):
 * source rank s, token i, k-th choice, with expert e = expert_ids[s][i][k].
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers into the memory of the current HIP device;
 *     arrays are dense, C-contiguous, in the shapes given.  bf16 is the 16-bit brain-float
 *     bit pattern; every token tensor below written "bf16" (x, ori_x, shared_x, expert_out,
 *     y, mode-0 expand_x) holds IEEE binary16 instead when cfg->token_dtype is
 *     MOE_TOKEN_F16, and y then rounds to binary16.  Device pointers should be 16-byte
 *     aligned for the vectorised kernels;
 *     unaligned pointers (or H not a multiple of 8) select slower element-wise kernels.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  Every
 *     call is asynchronous on that stream: it validates on the host, enqueues kernels and
 *     returns; outputs are valid in stream order.  No call synchronises the host, and no
 *     call allocates or frees memory: the caller owns every buffer and the stream.
 *   - A negative status other than MOE_ERR_DEVICE means nothing was enqueued (after
 *     MOE_ERR_DEVICE, kernels enqueued before the failing launch may still run and the
 *     outputs are undefined); moe_dc_last_error() then describes the
 *     problem (thread-local, valid until the next call on the same thread).
 */
#ifndef MOE_DC_H
#define MOE_DC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* a range, divisibility, pointer or size rule is broken   */
    MOE_ERR_UNSUPPORTED = -2,   /* allowed by the pages but not built (const experts)      */
    MOE_ERR_WORKSPACE = -3,     /* workspace missing or smaller than the query returned    */
    MOE_ERR_DEVICE = -4         /* a HIP runtime call failed                               */
} moe_status;

/* Element type of expand_x ([LLD] 约束说明 lists the types each quant mode allows). */
typedef enum {
    MOE_DTYPE_DEFAULT = 0,      /* the mode's default: bf16 (mode 0), int8 (modes 1, 2),
                                   E4M3 (modes 3, 4, 5)                                     */
    MOE_DTYPE_INT8 = 1,         /* modes 1, 2                                              */
    MOE_DTYPE_E4M3 = 2,         /* OCP E4M3 ("fn": bias 7, max 448); modes 2-5             */
    MOE_DTYPE_E5M2 = 3,         /* OCP E5M2 (bias 15, max 57344); modes 2-5                */
    MOE_DTYPE_E2M1 = 4          /* OCP E2M1 fp4 (max 6), two codes per byte, the element of
                                   even index in the low nibble; modes 4/5, H even          */
} moe_dtype;

/* Shape of the quantization scales tensor ([LLD] 约束说明: for mode 1 a scalar quant
 * coefficient, a row shared by every expert, or one row per expert; modes 2 and 3 take the
 * same shapes as smooth scales). */
typedef enum {
    MOE_SCALES_NONE = 0,        /* no scales tensor (modes 0, 2, 3, 4, 5)                  */
    MOE_SCALES_SCALAR = 1,      /* fp32 [1]                                                */
    MOE_SCALES_SHARED = 2,      /* fp32 [H], the same row for every expert                 */
    MOE_SCALES_PER_EXPERT = 3   /* fp32 [E][H]; the routed expert's row, so quantization is
                                   per pick                                                */
} moe_scales_kind;

/* Storage of the MX block scales (modes 4/5). */
typedef enum {
    MOE_SCALE_FP32 = 0,         /* fp32 2^shared_exp                                        */
    MOE_SCALE_E8M0 = 1,         /* one byte shared_exp + 127 ([SMP] 通信前量化 stores the MX
                                   scale as an E8M0 value)                                  */
    MOE_SCALE_FP32_RECIPROCAL = 2 /* fp32 2^-shared_exp, exact: the value that the [LLD]
                                   计算公式 of modes 4/5 writes out, 1.0 divided by the
                                   block's 2^shared_exp; the pad entry 0                     */
} moe_scale_format;

/* Element type of the tokens: x, ori_x, shared_x, expert_out, y and the mode-0 rows of
 * expand_x ([LLD] and [OPS] 参数说明: the token dtype is float16 or bfloat16). */
typedef enum {
    MOE_TOKEN_BF16 = 0,         /* bfloat16                                                */
    MOE_TOKEN_F16 = 1           /* IEEE binary16; y rounds to nearest even, overflow to inf */
} moe_token_dtype;

/* Bits of moe_dc_config.flags. */
typedef enum {
    /* moe_dispatch always runs the routing and the prefix sums as kernels of their own.  By
     * default a small batch (W*BS*K <= 2048 picks and E*W <= 4096, with the vectorised
     * scatter) computes them inside the scatter launch instead, one launch in place of
     * three; the results are identical either way. */
    MOE_DC_FLAG_SEPARATE_ROUTE = 1,
    /* moe_dispatch also counts the active picks whose expert id lies outside
     * [0, E + zero + copy) -- a contract violation the kernels otherwise skip silently -- and
     * stores the count as the int32 at byte 0 of the workspace (valid in stream order, until
     * the workspace is used again). */
    MOE_DC_FLAG_CHECK_IDS = 2
} moe_dc_flag;

/* Operator attributes ([OPS] 参数说明; [LLD] 约束说明).  One struct serves both calls; the
 * pages require the same values on every rank and for dispatch and its combine
 * ([OPS] 约束说明, cross-card consistency), which one struct gives for free.
 * Layout: sixteen int32 then one int64, 72 bytes, no padding. */
typedef struct {
    int32_t ep_world_size;          /* W, in [2, 768]                                        */
    int32_t moe_expert_num;         /* E, in (0, 1024], E % W == 0; L*W <= 2048               */
    int32_t bs;                     /* BS tokens per rank, in [1, 512]                        */
    int32_t hidden;                 /* H, in [1024, 8192]                                     */
    int32_t topk;                   /* K, in (0, 16], K <= E + zero + copy + const            */
    int32_t quant_mode;             /* 0 none, 1 static int8, 2 dynamic per token,
                                       3 dynamic per 128-element group, 4 MX, 5 MX clip       */
    int32_t zero_expert_num;        /* >= 0; ids [E, E+Z) are zero experts                    */
    int32_t copy_expert_num;        /* >= 0; ids [E+Z, E+Z+C) are copy experts               */
    int32_t const_expert_num;       /* must be 0 (its parameters are not on the pages)        */
    int32_t expert_token_nums_type; /* 0 = running sum over local experts, 1 = counts         */
    int32_t mask_kind;              /* 0 none, 1 per token [W][BS], 2 per pick [W][BS][K]     */
    int32_t out_dtype;              /* moe_dtype: mode 0 DEFAULT only; mode 1 DEFAULT/INT8;
                                       mode 2 DEFAULT/INT8/E4M3/E5M2; mode 3 DEFAULT/E4M3/
                                       E5M2; modes 4/5 DEFAULT/E4M3/E5M2/E2M1                */
    int32_t scales_kind;            /* moe_scales_kind: mode 1 SCALAR/SHARED/PER_EXPERT;
                                       modes 2, 3 any; modes 0, 4, 5 NONE                     */
    int32_t scale_format;           /* moe_scale_format: E8M0 and FP32_RECIPROCAL only with
                                       modes 4/5                                              */
    int32_t flags;                  /* moe_dc_flag bits; 0 for the defaults                   */
    int32_t token_dtype;            /* moe_token_dtype of x, ori_x, shared_x, expert_out, y
                                       and mode-0 expand_x: BF16 (0, the default) or F16      */
    int64_t expand_rows_capacity;   /* rows of expand_x / dynamic_scales / assist_info and of
                                       expert_out; must be >= W*BS*K                           */
} moe_dc_config;

/* Host-only check of every rule the pages state for the attributes ([OPS] 约束说明 and the
 * wrapper's checks under 调用说明; [LLD] 约束说明): the ranges above, E % W == 0,
 * L*W <= 2048, K <= E+Z+C+const, E+Z+C+const < INT32_MAX, capacity >= W*BS*K and < 2^31,
 * and the pairings of quant_mode with out_dtype, scales_kind and scale_format above.
 * Returns MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED.  Touches no device. */
moe_status moe_dc_validate(const moe_dc_config* cfg);

/* Scales per expand_x row for cfg->quant_mode (the dynamic_scales shape rule of [LLD]
 * 约束说明): 0 for modes 0 and 1, 1 for mode 2, Ceil(H, 128) for mode 3 and
 * Align2(Ceil(H, 32)) for modes 4/5.  Each scale is an fp32, or one byte with
 * MOE_SCALE_E8M0.  Returns -1 for an invalid config. */
int32_t moe_dc_scales_per_row(const moe_dc_config* cfg);

/* Workspace bytes moe_dispatch needs for this config (the pages' two-phase pattern:
 * query the workspace size, then execute; [OPS] 调用说明).  0 for an invalid config.
 * The workspace is scratch: its contents need no initialisation and are meaningless after
 * the call (except the checked-ids count of MOE_DC_FLAG_CHECK_IDS at byte 0); one workspace
 * must not be used by two dispatches that may run concurrently. */
size_t moe_dc_dispatch_workspace_bytes(const moe_dc_config* cfg);

/* moe_dispatch -- quantize, route and scatter every pick to its receiver's packed rows.
 *
 * Defined by: [DDD] §2.2 (index computation: per source rank, a pick's expand_idx is the
 * count of that rank's earlier picks, in row-major (token, pick) order, that chose the same
 * expert; the target rank is e / L rounded down and the local expert e % L); [DDD] §2.4
 * (receive side: the W x L count matrix is transposed and prefix-summed row-major into
 * ep_recv_count; expert_token_nums is its last column); [OPS] 功能说明 情形 1/2 and
 * [LLD] 计算公式 (quantization formulas of modes 0-5); [SMP] Dispatch 功能介绍
 * (each row carries its source triple, output as assist_info_for_combine).
 *
 * Quantization of a token x (x_fp32 = x widened to fp32, times the scales tensor if any):
 *   mode 1  codes = int8(x_fp32)
 *   mode 2  dyn = type_max / max|x_fp32| over the token; codes = type(x_fp32 * dyn);
 *           scale = 1/dyn (type_max 127 int8, 448 E4M3, 57344 E5M2)
 *   mode 3  as mode 2 for each group of 128 consecutive elements (the last may be short)
 *   mode 4  per 32-element block: shared_exp = floor(log2 max|x|) - emax, at least -127
 *           (emax 8 for E4M3, 15 for E5M2; an all-zero block takes -127)
 *   mode 5  per block: shared_exp = ceil(log2(max(max|x|, 1e-4) / type_max))
 *   modes 4/5: codes = fp8(x / 2^shared_exp); scale = 2^shared_exp (the dequant multiplier);
 *           E2M1 elements use emax 2 and type_max 6
 *
 * Inputs:
 *   x              bf16  [W][BS][H]   tokens of every source rank (finite values)
 *   expert_ids     int32 [W][BS][K]   picks; ids >= E are the special experts
 *   scales         fp32, shaped by cfg->scales_kind ([1], [H] or [E][H]); NULL iff
 *                  scales_kind is MOE_SCALES_NONE
 *   x_active_mask  uint8 [W][BS] (mask_kind 1) or [W][BS][K] (mask_kind 2), or NULL when
 *                  mask_kind is 0; nonzero = active.  An inactive pick is not dispatched.
 *   expert_scales  fp32 [W][BS][K] pick weights, or NULL; given exactly when expand_scales
 *                  is given (each routed row then carries its pick's weight)
 * Outputs (row = a receiver row in the packed layout below; cap = expand_rows_capacity):
 *   expand_x       [cap][H] bf16 (mode 0), [cap][H/2] bytes for E2M1 (two codes per byte),
 *                  else [cap][H] bytes: int8 or fp8 codes
 *   dynamic_scales [cap][moe_dc_scales_per_row(cfg)] fp32 (or bytes with MOE_SCALE_E8M0):
 *                  mode 2 one 1/dyn per row; mode 3 one 1/dyn per group; modes 4/5 one scale
 *                  per 32-element block (2^shared_exp, its E8M0 byte, or 2^-shared_exp, as
 *                  scale_format says) and 0 in the Align2 pad slot.  NULL allowed for
 *                  modes 0 and 1, which have no scales
 *   expand_idx     int32 [W][BS][K]   ordinal of each pick among its source rank's picks of
 *                  the same expert; -1 for inactive picks and special experts
 *   assist_info    int32 [cap][3]     (s, i, k) of the pick stored in each row
 *   ep_recv_count  int32 [W][L*W]     receiver r, entry j*W+s: inclusive running total of
 *                  the rows r receives, over (local expert j, source s) in that order
 *   expert_token_nums int64 [W][L]    type 1: rows per local expert; type 0: running sum
 *   recv_offsets   int64 [W+1]        first row of each receiver; [W] = total routed rows
 *   expand_scales  fp32 [cap] or NULL: each row's pick weight ([OPS] 参数说明,
 *                  expand_scales_out: the weight travels with its token)
 *   workspace      moe_dc_dispatch_workspace_bytes(cfg) bytes, 4-byte aligned
 * Packed layout: receiver r owns rows [recv_offsets[r], recv_offsets[r+1]); inside, rows go
 * by local expert, then source rank, then expand_idx.  So the whole buffer is one stable sort
 * of the routed picks by (expert, s, i, k).  Rows at or past recv_offsets[W] are not written.
 * Numerics: every fp32 operation is a single IEEE binary32 operation rounded to nearest
 * even, in the order of the formulas; int8 codes round half to even and saturate at +-127
 * (NaN -> 0); fp8 codes round to nearest even and saturate at +-448 (E4M3) or +-57344
 * (E5M2); in modes 2/3 an all-zero segment gives codes 0 and scale 0; fp32 subnormals are
 * kept.  The results are deterministic: identical inputs give identical bytes.
 * Errors: host validation first (MOE_ERR_INVALID_ARG / _UNSUPPORTED / _WORKSPACE); a HIP
 * launch failure gives MOE_ERR_DEVICE.  Out-of-range expert ids are a contract violation:
 * the kernels never access memory out of bounds for them and treat such picks as not
 * dispatched; MOE_DC_FLAG_CHECK_IDS counts them.  A per-token mask needs no particular order (the pages ask for trues before
 * falses; any order works here). */
moe_status moe_dispatch(const moe_dc_config* cfg,
                        const void* x, const int32_t* expert_ids,
                        const float* scales, const uint8_t* x_active_mask,
                        const float* expert_scales,
                        void* expand_x, void* dynamic_scales, int32_t* expand_idx,
                        int32_t* assist_info, int32_t* ep_recv_count,
                        int64_t* expert_token_nums, int64_t* recv_offsets,
                        float* expand_scales,
                        void* workspace, size_t workspace_bytes, void* stream);

/* moe_dispatch_no_workspace -- moe_dispatch without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It runs the same kernels and writes the same outputs as
 * moe_dispatch; its workspace is a 1 MiB array in the library's own device memory, one per
 * GPU, held from the library's load until the process ends.
 *
 * Arguments: as for moe_dispatch, less workspace and workspace_bytes.
 * Limits and errors: a config whose moe_dc_dispatch_workspace_bytes exceeds 1 MiB
 * (E * W above about 260,000 counts) returns MOE_ERR_WORKSPACE, and MOE_DC_FLAG_CHECK_IDS
 * (whose count lands in the caller's workspace) returns MOE_ERR_INVALID_ARG; both are checked
 * on the host before anything is enqueued.  The first call on a device looks up that device's
 * copy of the array (MOE_ERR_DEVICE if the lookup fails).  Nothing is allocated or freed.
 * Every call on one GPU uses the same array: calls that may run concurrently on one GPU
 * (other streams, other threads) race and must be ordered by the caller. */
moe_status moe_dispatch_no_workspace(const moe_dc_config* cfg,
                                     const void* x, const int32_t* expert_ids,
                                     const float* scales, const uint8_t* x_active_mask,
                                     const float* expert_scales,
                                     void* expand_x, void* dynamic_scales, int32_t* expand_idx,
                                     int32_t* assist_info, int32_t* ep_recv_count,
                                     int64_t* expert_token_nums, int64_t* recv_offsets,
                                     float* expand_scales, void* stream);

/* moe_combine -- gather each token's K expert outputs and form their weighted sum.
 *
 * Defined by: [DDD] §3.4 (a pick's expert output sits at its rank's window + the expert's
 * offset + expand_idx; the K outputs are weighted and summed back to the token); [SMP]
 * Combine 功能介绍 (each expert row times its expert scale, accumulated in fp32, then cast
 * down); [LLD] 计算公式 特殊专家场景 (a zero expert outputs 0, a copy expert outputs ori_x).
 *
 * Inputs:
 *   expert_out     bf16 [cap][H]      expert outputs, row-aligned with dispatch's expand_x
 *   expert_ids, expand_idx, ep_recv_count, recv_offsets: as produced by moe_dispatch for
 *                  this config (the addressing uses exactly these)
 *   expert_scales  fp32 [W][BS][K]    weight of each pick
 *   x_active_mask  as for moe_dispatch (inactive picks contribute nothing)
 *   ori_x          bf16 [W][BS][H]    dispatch's x; required iff copy_expert_num > 0
 * Output:
 *   y              bf16 [W][BS][H]    y[s][i] = bf16_rne( sum over active picks in k order of
 *                  w * expert_row ), accumulated in fp32 starting from +0 with one multiply
 *                  and one add per pick (zero experts add nothing); all-inactive tokens -> +0
 * Errors: as for moe_dispatch; ori_x NULL with copy experts is MOE_ERR_INVALID_ARG.
 * Needs no workspace. */
moe_status moe_combine(const moe_dc_config* cfg,
                       const void* expert_out, const int32_t* expert_ids,
                       const int32_t* expand_idx, const float* expert_scales,
                       const int32_t* ep_recv_count, const int64_t* recv_offsets,
                       const uint8_t* x_active_mask, const void* ori_x, void* y,
                       void* stream);

/* Workspace bytes moe_combine_scatter needs: one int32 per pick slot (W*BS*K), rounded up
 * to 256.  0 for an invalid config.  Scratch, as for dispatch. */
size_t moe_dc_combine_scatter_workspace_bytes(const moe_dc_config* cfg);

/* moe_combine_scatter -- the scatter-back combine: rows return to their sources by their
 * source triples, then each token sums its K slots and adds the shared expert's output.
 *
 * Defined by: [SMP] Combine 功能介绍 计算步骤 and 源码实现: each expert-side row r is sent back
 * using its triple (s, i, k) = assist_info[r] to offset epOffset = i * K + k of source rank s;
 * the source then multiplies each of a token's K results by its expert scale, sums them in
 * fp32 and adds the shared expert's result.  All ranks share this GPU's memory, so a slot
 * stores the row's index (in the workspace) and the sum reads the row through it: the same
 * values as copying the row, without moving its bytes twice.
 *
 * Inputs:
 *   expert_out     bf16 [cap][H]      expert outputs, row-aligned with expand_x
 *   assist_info    int32 [cap][3]     from moe_dispatch; rows [0, recv_offsets[W]) are sent
 *   recv_offsets   int64 [W+1]        from moe_dispatch
 *   expert_ids     int32 [W][BS][K]   which picks are routed, zero or copy experts
 *   expert_scales  fp32 [W][BS][K]    the source's pick weights
 *   x_active_mask  as for moe_dispatch
 *   ori_x          bf16 [W][BS][H]    required iff copy_expert_num > 0
 *   shared_x       bf16 [W][BS][H]    the shared expert's output per token, or NULL
 * Output:
 *   y              bf16 [W][BS][H] = bf16_rne( sum over active picks in k order of w * row,
 *                  then + shared_x ), accumulated in fp32 from +0
 * Errors: as for moe_combine; a workspace smaller than the query is MOE_ERR_WORKSPACE. */
moe_status moe_combine_scatter(const moe_dc_config* cfg, const void* expert_out,
                               const int32_t* assist_info, const int64_t* recv_offsets,
                               const int32_t* expert_ids, const float* expert_scales,
                               const uint8_t* x_active_mask, const void* ori_x,
                               const void* shared_x, void* y, void* workspace,
                               size_t workspace_bytes, void* stream);

/* moe_combine_quantize -- expert-side int8 block quantization of the expert outputs, the
 * compression the pages apply before the combine's return transfer.
 *
 * Defined by: [SMP] 通信前量化 (Combine 的 INT8 block 量化): each expert-output row is cut into
 * blocks of 8 elements (32 bytes of fp32); per block scale = amax * (1/127) (the reciprocal of
 * 127 rounded once to fp32), and each code = int8(fp16(x / scale)), where the division is one
 * IEEE fp32 division and each narrowing rounds to nearest even (int8 saturates at +-127; an
 * all-zero block gives codes 0 and scale 0).
 *
 * Inputs:
 *   expert_out     bf16 [cap][H]      as for moe_combine
 *   recv_offsets   int64 [W+1]        from moe_dispatch; rows [0, recv_offsets[W]) are coded
 * Outputs:
 *   codes          int8 [cap][H]
 *   block_scales   fp32 [cap][Ceil(H, 8)]
 * Rows at or past recv_offsets[W] are not written.  Errors as for moe_combine. */
moe_status moe_combine_quantize(const moe_dc_config* cfg, const void* expert_out,
                                const int64_t* recv_offsets, int8_t* codes,
                                float* block_scales, void* stream);

/* moe_combine_int8 -- moe_combine over block-quantized expert outputs.
 *
 * Defined by: moe_combine's definition with each routed pick's row dequantized first
 * ([SMP] 通信前量化: int8 -> fp16 -> float, both exact, times the block's scale, one fp32
 * multiply); zero experts add nothing, copy experts add w * ori_x (ori_x is not quantized).
 *
 * Inputs: codes and block_scales as written by moe_combine_quantize; the other arguments as
 * for moe_combine.  Output: y bf16 [W][BS][H] = bf16_rne( sum over active picks in k order
 * of w * (code * scale) ), accumulated in fp32 from +0.  Errors as for moe_combine. */
moe_status moe_combine_int8(const moe_dc_config* cfg, const int8_t* codes,
                            const float* block_scales, const int32_t* expert_ids,
                            const int32_t* expand_idx, const float* expert_scales,
                            const int32_t* ep_recv_count, const int64_t* recv_offsets,
                            const uint8_t* x_active_mask, const void* ori_x, void* y,
                            void* stream);

/* Text of the last non-OK status on this thread ("" if none). */
const char* moe_dc_last_error(void);

/* Library version string. */
const char* moe_dc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DC_H */
