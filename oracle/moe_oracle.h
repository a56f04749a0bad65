/*
 * moe_oracle.h -- plain, slow, single-threaded CPU oracle for MoE dispatch/combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or call
 * this code: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
 * It shares no header, helper, table or constant with the HIP library.
 *
 * Pages cited (by title; sections as numbered on each page):
 *   [DDD] "MoeDistributeDispatch和MoeDistributeCombine算子设计介绍" (gitcode design doc, Atlas A2)
 *   [LLD] "low_latency_dispatch" (hiascend API doc), sections 计算公式 and 约束说明
 *   [OPS] "CANN ops-transformer 算子解析：MoeDistributeDispatchV3 的 EP 域 Token 分发与动态量化通信实现"
 *         (mwwr.cn article), sections 功能说明, 参数说明, 约束说明, 接口级量化模式扩展
 *   [SMP] "CANN MoE Dispatch/Combine 通信算子性能优化实践：Kernel 直调与 ACL SHMEM 实现专家分发与聚合"
 *         (lqnn.cn article), sections Dispatch 功能介绍, Combine 功能介绍, 通信前量化
 *
 * Conventions: all pointers are host pointers; token values (bf16 or binary16, by the
 * config's token_dtype) travel as uint16_t bit patterns;
 * arrays are C-contiguous in the shapes stated at each function.  Return 0 on success,
 * a negative value on a contract violation (the oracle refuses rather than guesses).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t W;                      /* logical EP ranks                                   */
    int32_t E;                      /* routed experts; L = E / W per rank                 */
    int32_t BS;                     /* tokens per source rank                             */
    int32_t H;                      /* hidden size                                        */
    int32_t K;                      /* picks per token                                    */
    int32_t quant_mode;             /* 0 none, 1 static, 2 per token, 3 per 128-group,
                                       4 MX, 5 MX clip                                      */
    int32_t zero_expert_num;        /* ids [E, E+Z) are zero experts                      */
    int32_t copy_expert_num;        /* ids [E+Z, E+Z+C) are copy experts                  */
    int32_t expert_token_nums_type; /* 0 inclusive cumsum, 1 per-expert counts            */
    int32_t mask_kind;              /* 0 none, 1 per token [W][BS], 2 per pair [W][BS][K] */
    int32_t out_dtype;              /* 0 the mode's default, else one of ORACLE_CODE_*     */
    int32_t scales_kind;            /* 0 none, 1 scalar (1,), 2 shared (H,), 3 per expert  */
    int32_t scale_format;           /* 0 fp32 scales, 1 E8M0 bytes, 2 fp32 1/scale
                                       (1 and 2: modes 4/5 only)                             */
    int32_t token_dtype;            /* token elements (x, ori_x, expert outputs, y): 0 bf16,
                                       1 IEEE binary16                                      */
} oracle_cfg;

/* element types of expand_x */
#define ORACLE_CODE_BF16 0
#define ORACLE_CODE_INT8 1
#define ORACLE_CODE_E4M3 2
#define ORACLE_CODE_E5M2 3
#define ORACLE_CODE_E2M1 4              /* fp4, two codes per byte (modes 4/5, even H) */

/* scalar helpers (each written from its definition) */
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);
uint8_t  oracle_e4m3_from_f32(float v);
float    oracle_e4m3_to_f32(uint8_t code);
uint8_t  oracle_e5m2_from_f32(float v);
float    oracle_e5m2_to_f32(uint8_t code);
uint8_t  oracle_e2m1_from_f32(float v);
float    oracle_e2m1_to_f32(uint8_t code);
int32_t  oracle_code_row_bytes(int32_t code_type, int32_t H);
int8_t   oracle_int8_from_f32(float v);
uint8_t  oracle_e8m0_from_scale(float s);
int32_t  oracle_mx_scale_count(int32_t H);
int32_t  oracle_code_type(int32_t quant_mode, int32_t out_dtype);
int32_t  oracle_scale_count(int32_t quant_mode, int32_t H);

/* IEEE binary16 (fp16) conversions */
uint16_t oracle_f32_to_f16(float f);
float    oracle_f16_to_f32(uint16_t h);
int8_t   oracle_int8_from_f16(uint16_t h);

/* per-row quantization */
void oracle_quant_int8_row(const uint16_t* x, const float* smooth_or_null, int32_t H,
                           int8_t* q, float* scale);
void oracle_quant_mx_row(const uint16_t* x, int32_t H, int32_t clip, uint8_t* codes,
                         float* scales);
int32_t oracle_quant_row(int32_t quant_mode, int32_t code_type, const uint16_t* x,
                         const float* pre, int32_t pre_len, int32_t H, void* codes,
                         float* scales);
/* Same, with the row's elements bf16 (token_dtype 0) or binary16 (1). */
int32_t oracle_quant_row_tok(int32_t token_dtype, int32_t quant_mode, int32_t code_type, const uint16_t* x,
                         const float* pre, int32_t pre_len, int32_t H, void* codes,
                         float* scales);

/* routing, receive counts, destination rows */
int32_t oracle_route(const oracle_cfg* c, const int32_t* expert_ids, const uint8_t* mask,
                     int32_t* cnt, int32_t* expand_idx);
int32_t oracle_recv_counts(const oracle_cfg* c, const int32_t* cnt, int32_t* ep_recv_count,
                           int64_t* expert_token_nums, int64_t* recv_offsets);
int64_t oracle_dest_row(const oracle_cfg* c, const int32_t* ep_recv_count,
                        const int64_t* recv_offsets, int32_t s, int32_t e, int32_t ordinal);

/* whole dispatch and combine */
int32_t oracle_dispatch(const oracle_cfg* c, const uint16_t* x, const int32_t* expert_ids,
                        const float* scales_or_null, const uint8_t* mask, void* expand_x,
                        void* dynamic_scales, int32_t* expand_idx, int32_t* assist_info,
                        int32_t* ep_recv_count, int64_t* expert_token_nums,
                        int64_t* recv_offsets, int32_t* cnt_scratch);
int32_t oracle_combine_token(const oracle_cfg* c, const uint16_t* expert_out,
                             const int32_t* expert_ids, const int32_t* expand_idx,
                             const float* expert_scales, const int32_t* ep_recv_count,
                             const int64_t* recv_offsets, const uint8_t* mask,
                             const uint16_t* ori_x, int32_t s, int32_t i, float* acc_scratch,
                             uint16_t* y_row);
/* combine-side int8 block quantization (expert side) and the int8 combine (source side) */
int32_t oracle_combine_block_count(int32_t H);
void oracle_combine_quant_row(const uint16_t* row, int32_t H, int8_t* q, float* scales);
void oracle_combine_quant_row_tok(int32_t token_dtype, const uint16_t* row, int32_t H, int8_t* q,
                                  float* scales);
void oracle_combine_dequant_row(const int8_t* q, const float* scales, int32_t H, float* out);
int32_t oracle_combine_quantize(const oracle_cfg* c, const uint16_t* expert_out,
                                const int64_t* recv_offsets, int8_t* codes, float* scales);
int32_t oracle_combine_int8_token(const oracle_cfg* c, const int8_t* codes, const float* scales,
                                  const int32_t* expert_ids, const int32_t* expand_idx,
                                  const float* expert_scales, const int32_t* ep_recv_count,
                                  const int64_t* recv_offsets, const uint8_t* mask,
                                  const uint16_t* ori_x, int32_t s, int32_t i,
                                  float* acc_scratch, float* row_scratch, uint16_t* y_row);
int32_t oracle_combine_int8(const oracle_cfg* c, const int8_t* codes, const float* scales,
                            const int32_t* expert_ids, const int32_t* expand_idx,
                            const float* expert_scales, const int32_t* ep_recv_count,
                            const int64_t* recv_offsets, const uint8_t* mask,
                            const uint16_t* ori_x, uint16_t* y, float* acc_scratch,
                            float* row_scratch);
int32_t oracle_expand_scales(const oracle_cfg* c, const int32_t* assist_info,
                             const int64_t* recv_offsets, const float* expert_scales,
                             float* expand_scales);
int32_t oracle_combine_scatter(const oracle_cfg* c, const uint16_t* expert_out,
                               const int32_t* assist_info, const int64_t* recv_offsets,
                               const int32_t* expert_ids, const float* expert_scales,
                               const uint8_t* mask, const uint16_t* ori_x,
                               const uint16_t* shared_x, uint16_t* y,
                               uint16_t* window_scratch, float* acc_scratch);
int32_t oracle_combine(const oracle_cfg* c, const uint16_t* expert_out,
                       const int32_t* expert_ids, const int32_t* expand_idx,
                       const float* expert_scales, const int32_t* ep_recv_count,
                       const int64_t* recv_offsets, const uint8_t* mask,
                       const uint16_t* ori_x, uint16_t* y, float* acc_scratch);

#ifdef __cplusplus
}
#endif
#endif
