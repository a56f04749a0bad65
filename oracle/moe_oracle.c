/*
 * moe_oracle.c -- plain CPU oracle for MoE dispatch/combine (see moe_oracle.h for the pages).
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg; never by the product path.  Built with gcc -O2 -ffp-contract=off and no
 * fast-math, so every float operation below is one IEEE-754 binary32 operation rounded to
 * nearest-even, in the order written.
 *
 * Every function restates what the pages define, in the pages' order.  Where a page is
 * silent or garbled the reading taken is named inline (R1..R12) and listed with its reason
 * in the design notes of the repository.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------- */
/* scalar helpers                                                                        */
/* ------------------------------------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32 pattern: widening is exact. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Narrowing to bf16 by round-to-nearest, ties to even, keeping NaN a quiet NaN.
 * The rounding is done on the exact value: the dropped 16 bits are compared with the
 * halfway point 0x8000; above rounds up, below truncates, equal goes to the even pattern.
 * A carry out of the mantissa correctly steps into the exponent (and to infinity). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t drop = u & 0xFFFFu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

/* OCP E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the
 * all-ones pattern S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 * Subnormals are m * 2^-9 for m = 1..7. */
float oracle_e4m3_to_f32(uint8_t code)
{
    int sign = code & 0x80;
    int ex = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (ex == 0xF && m == 0x7) return NAN;
    if (ex == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, ex - 7);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest E4M3 value, ties to the even code, saturating any
 * magnitude >= 448 to +-448 (reading R6: the pages leave MX overflow unsaid; the MX
 * convention is to clamp to the largest finite element value).  Sign is kept, so a
 * negative value that rounds to zero gives the negative-zero code 0x80.
 * Method: work in double, where every step below is exact.  Pick the spacing (quantum)
 * of E4M3 values in the binade of |v| (2^-9 throughout the subnormal range), take the
 * nearest integer multiple of it with nearbyint (ties-to-even under the default rounding
 * mode; an even multiple is exactly an even mantissa code), then encode. */
uint8_t oracle_e4m3_from_f32(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    double quantum;
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        int ex;
        frexp(a, &ex);               /* a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex-1 */
        quantum = ldexp(1.0, (ex - 1) - 3);
    }
    double n = nearbyint(a / quantum);
    double r = n * quantum;          /* representable, <= 448 because a < 448 */
    uint8_t code;
    if (r < ldexp(1.0, -6)) {
        code = (uint8_t)(r / ldexp(1.0, -9));          /* 0..8; 8 is exactly 2^-6 = 0x08 */
    } else {
        int ex;
        double m = frexp(r, &ex);    /* r = m * 2^ex, m in [0.5, 1) */
        int e2 = ex - 1;             /* r = (2m) * 2^e2, 2m in [1, 2) */
        int mant = (int)((2.0 * m - 1.0) * 8.0);       /* exact: 2m has 3 fraction bits */
        code = (uint8_t)(((e2 + 7) << 3) | mant);
    }
    return (uint8_t)(sign | code);
}

/* MX scales per row: one per 32-element block, padded to an even count (Align2 of
 * Ceil(H, 32)) as the dynamic_scales shape rule for quant modes 4/5 states ([LLD] 约束说明). */
int32_t oracle_mx_scale_count(int32_t H)
{
    int32_t nb = (H + 31) / 32;
    return nb + (nb & 1);
}

/* ------------------------------------------------------------------------------------- */
/* quantization                                                                          */
/* ------------------------------------------------------------------------------------- */

/* Per-token dynamic int8 quantization, quant_mode 2 ([OPS] 功能说明 情形 2; [LLD] 计算公式,
 * quant_mode=2):
 *   x_fp32 = CastToFp32(x), times the smooth-scale row if one is given
 *   dyn    = 127 / max|x_fp32|           (127 is int8's largest value)
 *   q      = CastToInt8(x_fp32 * dyn)
 *   scale  = 1.0 / dyn                   (sent with the row; dequant is q * scale)
 * Reading R4: the int8 cast rounds half to even.  Reading R5: the cast saturates to
 * [-127, 127] and maps NaN to 0; with an all-zero row dyn = 127/0 = +inf, every product is
 * 0*inf = NaN -> 0, and scale = 1/inf = 0. */
void oracle_quant_int8_row(const uint16_t* x, const float* smooth_or_null, int32_t H,
                           int8_t* q, float* scale)
{
    float* f = (float*)malloc((size_t)H * sizeof(float));
    for (int32_t h = 0; h < H; ++h) {
        f[h] = oracle_bf16_to_f32(x[h]);
        if (smooth_or_null) f[h] = f[h] * smooth_or_null[h];
    }
    float amax = 0.0f;
    for (int32_t h = 0; h < H; ++h)
        if (fabsf(f[h]) > amax) amax = fabsf(f[h]);
    float dyn = 127.0f / amax;
    for (int32_t h = 0; h < H; ++h) {
        float v = f[h] * dyn;
        float r;
        if (isnan(v)) r = 0.0f;
        else {
            r = nearbyintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
        }
        q[h] = (int8_t)r;
    }
    *scale = 1.0f / dyn;
    free(f);
}

/* floor(log2(a)) for a finite a > 0, exactly: frexpf gives a = m * 2^ex with m in [0.5,1). */
static int ilog2_floor(float a)
{
    int ex;
    frexpf(a, &ex);
    return ex - 1;
}

/* MX quantization of one row, in blocks of 32 elements (the last block may be short).
 * quant_mode 4 ([LLD] 计算公式, quant_mode=4; [OPS] 接口级量化模式扩展):
 *   shared_exp = floor(log2(max|x| over the block)) - emax,  emax = 8 for E4M3
 *   q = Cast(x / 2^shared_exp, e4m3)
 * Reading R7: max(x) is the block's absolute maximum.  Reading R8: an all-zero block takes
 * shared_exp = -127, and shared_exp is clamped below at -127 (the E8M0 range).
 * quant_mode 5, the clip variant ([LLD] 计算公式, quant_mode=5):
 *   max_abs_clamp = max(max|x|, 1e-4);  shared_exp = ceil(log2(max_abs_clamp / 448))
 *   q = CastToFp8(x / 2^shared_exp)
 * Reading R9: max_abs_clamp / 448 is one fp32 division and its ceil(log2) is taken exactly.
 * Reading R10: the scale written for each block is 2^shared_exp, the dequant multiplier
 * (codes * scale ~ x).  Pad entries of the Align2 layout are 0. */
void oracle_quant_mx_row(const uint16_t* x, int32_t H, int32_t clip, uint8_t* codes,
                         float* scales)
{
    int32_t nb = (H + 31) / 32;
    int32_t ns = oracle_mx_scale_count(H);
    for (int32_t b = 0; b < nb; ++b) {
        int32_t h0 = b * 32;
        int32_t h1 = h0 + 32 < H ? h0 + 32 : H;
        float amax = 0.0f;
        for (int32_t h = h0; h < h1; ++h) {
            float a = fabsf(oracle_bf16_to_f32(x[h]));
            if (a > amax) amax = a;
        }
        int se;
        if (!clip) {
            if (amax == 0.0f) se = -127;
            else se = ilog2_floor(amax) - 8;
            if (se < -127) se = -127;
        } else {
            float c = amax > 1e-4f ? amax : 1e-4f;
            float v = c / 448.0f;
            int ex;
            float m = frexpf(v, &ex);  /* v = m * 2^ex; v is a power of two iff m == 0.5 */
            se = (m == 0.5f) ? ex - 1 : ex;
        }
        float sc = ldexpf(1.0f, se);   /* 2^-127 is a binary32 subnormal: exact */
        for (int32_t h = h0; h < h1; ++h) {
            float v = oracle_bf16_to_f32(x[h]) / sc;
            codes[h] = oracle_e4m3_from_f32(v);
        }
        scales[b] = sc;
    }
    for (int32_t b = nb; b < ns; ++b) scales[b] = 0.0f;
}

/* ------------------------------------------------------------------------------------- */
/* routing                                                                               */
/* ------------------------------------------------------------------------------------- */

static int pair_active(const oracle_cfg* c, const uint8_t* mask, int32_t s, int32_t i, int32_t k)
{
    if (c->mask_kind == 0 || mask == NULL) return 1;
    if (c->mask_kind == 1) return mask[(size_t)s * c->BS + i] != 0;
    return mask[((size_t)s * c->BS + i) * c->K + k] != 0;
}

/* Index computation ([DDD] §2.2.2 索引计算流程), run for every source rank s.  The pairs
 * (i, k) of expert_ids are walked row-major (token i outer, pick k inner); for a routed
 * pair with expert e the ordinal is the running count of earlier pairs of rank s that
 * went to e, after which that count is incremented.
 * Reading R1: the target rank is e / L rounded down (the page's "ceil" contradicts its own
 * local index e % L).  Reading R2: the count belongs to the source rank (the combine
 * address of [DDD] §3.4.2 needs exactly this).  Reading R3: inactive pairs ([OPS] 参数说明,
 * x_active_mask) and special experts ([LLD] 特殊专家场景) are not dispatched and get -1.
 *   cnt        [W][E]     count of routed pairs from source s to expert e
 *   expand_idx [W][BS][K] ordinal, or -1 */
int32_t oracle_route(const oracle_cfg* c, const int32_t* expert_ids, const uint8_t* mask,
                     int32_t* cnt, int32_t* expand_idx)
{
    const int32_t id_end = c->E + c->zero_expert_num + c->copy_expert_num;
    memset(cnt, 0, (size_t)c->W * c->E * sizeof(int32_t));
    for (int32_t s = 0; s < c->W; ++s)
        for (int32_t i = 0; i < c->BS; ++i)
            for (int32_t k = 0; k < c->K; ++k) {
                size_t p = ((size_t)s * c->BS + i) * c->K + k;
                int32_t e = expert_ids[p];
                if (e < 0 || e >= id_end) return -1;
                if (!pair_active(c, mask, s, i, k) || e >= c->E) {
                    expand_idx[p] = -1;
                    continue;
                }
                expand_idx[p] = cnt[(size_t)s * c->E + e];
                cnt[(size_t)s * c->E + e] += 1;
            }
    return 0;
}

/* Receive-side metadata ([DDD] §2.4.1-2.4.2).  Receiver r sees the W x L matrix
 * M_r(s, j) = cnt[s][r*L + j]; ep_recv_count is its transpose (L x W) followed by a
 * row-major running sum, so entry j*W + s is the inclusive total over (j', s') <= (j, s)
 * in that order.  expert_token_nums is the last column of that array (type 0, a running
 * sum over experts) or the plain per-expert totals (type 1) ([OPS] 参数说明,
 * expert_token_nums_type).  recv_offsets places each receiver's rows one after another.
 *   ep_recv_count     [W][L*W] int32
 *   expert_token_nums [W][L]   int64
 *   recv_offsets      [W+1]    int64 */
int32_t oracle_recv_counts(const oracle_cfg* c, const int32_t* cnt, int32_t* ep_recv_count,
                           int64_t* expert_token_nums, int64_t* recv_offsets)
{
    const int32_t W = c->W, L = c->E / c->W;
    recv_offsets[0] = 0;
    for (int32_t r = 0; r < W; ++r) {
        int64_t run = 0;
        for (int32_t j = 0; j < L; ++j) {
            int64_t per_expert = 0;
            for (int32_t s = 0; s < W; ++s) {
                int32_t m = cnt[(size_t)s * c->E + (size_t)r * L + j];
                run += m;
                per_expert += m;
                ep_recv_count[(size_t)r * L * W + (size_t)j * W + s] = (int32_t)run;
            }
            expert_token_nums[(size_t)r * L + j] =
                c->expert_token_nums_type == 0 ? run : per_expert;
        }
        recv_offsets[r + 1] = recv_offsets[r] + run;
    }
    return 0;
}

/* Destination row of a routed pair in the packed expand_x: receiver r's block starts at
 * recv_offsets[r]; inside it the (expert j, source s) segment starts at the running total
 * just before it, which is ep_recv_count_r[j*W + s - 1], or 0 for the very first segment
 * ([DDD] §3.2.2, the prefix-sum matrix example and its start-position rule; [DDD] §3.4.2
 * TokenAddr = rank window + expert offset + expandIdx); the pair's ordinal follows. */
int64_t oracle_dest_row(const oracle_cfg* c, const int32_t* ep_recv_count,
                        const int64_t* recv_offsets, int32_t s, int32_t e, int32_t ordinal)
{
    const int32_t W = c->W, L = c->E / c->W;
    int32_t r = e / L, j = e % L;
    int64_t flat = (int64_t)j * W + s;
    int64_t base = flat == 0 ? 0 : ep_recv_count[(size_t)r * L * W + flat - 1];
    return recv_offsets[r] + base + ordinal;
}

/* Full dispatch: route, count, then write each routed pair's payload at its destination
 * row, with the source triple (s, i, k) ([SMP] Dispatch 功能介绍, 计算步骤: the triple
 * travels with the quantized token and comes out as assist_info_for_combine).
 *   mode 0 ([LLD] quant_mode=0): the bf16 row is moved unchanged; no scales.
 *   mode 2: int8 row + one fp32 scale; the smooth-scale row is the routed expert's
 *           ([LLD] quant_mode 约束: shape (num_experts, H)), so quantization is per pair.
 *   mode 4/5: E4M3 codes + Align2(Ceil(H,32)) fp32 scales per row.
 *   expand_x [cap][H] (uint16 bf16 patterns for mode 0, else bytes);
 *   dynamic_scales [cap] or [cap][scale count]; assist_info [cap][3]. */
int32_t oracle_dispatch(const oracle_cfg* c, const uint16_t* x, const int32_t* expert_ids,
                        const float* smooth_or_null, const uint8_t* mask, void* expand_x,
                        float* dynamic_scales, int32_t* expand_idx, int32_t* assist_info,
                        int32_t* ep_recv_count, int64_t* expert_token_nums,
                        int64_t* recv_offsets, int32_t* cnt_scratch)
{
    const int32_t H = c->H;
    if (c->quant_mode != 0 && c->quant_mode != 2 && c->quant_mode != 4 && c->quant_mode != 5)
        return -2;
    if (smooth_or_null && c->quant_mode != 2) return -3;
    if (oracle_route(c, expert_ids, mask, cnt_scratch, expand_idx) != 0) return -1;
    oracle_recv_counts(c, cnt_scratch, ep_recv_count, expert_token_nums, recv_offsets);
    const int32_t ns = oracle_mx_scale_count(H);
    for (int32_t s = 0; s < c->W; ++s)
        for (int32_t i = 0; i < c->BS; ++i)
            for (int32_t k = 0; k < c->K; ++k) {
                size_t p = ((size_t)s * c->BS + i) * c->K + k;
                int32_t ord = expand_idx[p];
                if (ord < 0) continue;
                int32_t e = expert_ids[p];
                int64_t row = oracle_dest_row(c, ep_recv_count, recv_offsets, s, e, ord);
                const uint16_t* xr = x + ((size_t)s * c->BS + i) * H;
                if (c->quant_mode == 0) {
                    memcpy((uint16_t*)expand_x + (size_t)row * H, xr, (size_t)H * 2);
                } else if (c->quant_mode == 2) {
                    const float* sm = smooth_or_null ? smooth_or_null + (size_t)e * H : NULL;
                    oracle_quant_int8_row(xr, sm, H, (int8_t*)expand_x + (size_t)row * H,
                                          &dynamic_scales[row]);
                } else {
                    oracle_quant_mx_row(xr, H, c->quant_mode == 5,
                                        (uint8_t*)expand_x + (size_t)row * H,
                                        dynamic_scales + (size_t)row * ns);
                }
                assist_info[(size_t)row * 3 + 0] = s;
                assist_info[(size_t)row * 3 + 1] = i;
                assist_info[(size_t)row * 3 + 2] = k;
            }
    return 0;
}

/* ------------------------------------------------------------------------------------- */
/* combine                                                                               */
/* ------------------------------------------------------------------------------------- */

/* Combine for one source token ([DDD] §3.4.2 加权求和: locate each pick's expert output
 * with the TokenAddr rule, weight it, sum; [SMP] Combine 功能介绍: each expert row is
 * multiplied by its expert scale and accumulated in fp32, then cast down).  Special
 * experts ([LLD] 特殊专家场景): a zero expert's output is 0, a copy expert's is ori_x.
 * Reading R11: picks are summed in k order, as one fp32 multiply then one fp32 add each
 * (zero experts and inactive picks add nothing), starting from +0; the result is rounded
 * to bf16.  A token with no active pick therefore gives +0. */
int32_t oracle_combine_token(const oracle_cfg* c, const uint16_t* expert_out,
                             const int32_t* expert_ids, const int32_t* expand_idx,
                             const float* expert_scales, const int32_t* ep_recv_count,
                             const int64_t* recv_offsets, const uint8_t* mask,
                             const uint16_t* ori_x, int32_t s, int32_t i, float* acc,
                             uint16_t* y_row)
{
    const int32_t H = c->H;
    const int32_t zero_end = c->E + c->zero_expert_num;
    const int32_t copy_end = zero_end + c->copy_expert_num;
    for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
    for (int32_t k = 0; k < c->K; ++k) {
        size_t p = ((size_t)s * c->BS + i) * c->K + k;
        if (!pair_active(c, mask, s, i, k)) continue;
        int32_t e = expert_ids[p];
        float w = expert_scales[p];
        if (e < 0 || e >= copy_end) return -1;
        if (e < c->E) {
            int32_t ord = expand_idx[p];
            if (ord < 0) return -1;
            int64_t row = oracle_dest_row(c, ep_recv_count, recv_offsets, s, e, ord);
            const uint16_t* src = expert_out + (size_t)row * H;
            for (int32_t h = 0; h < H; ++h) {
                float t = w * oracle_bf16_to_f32(src[h]);
                acc[h] = acc[h] + t;
            }
        } else if (e < zero_end) {
            continue;
        } else {
            if (ori_x == NULL) return -1;
            const uint16_t* src = ori_x + ((size_t)s * c->BS + i) * H;
            for (int32_t h = 0; h < H; ++h) {
                float t = w * oracle_bf16_to_f32(src[h]);
                acc[h] = acc[h] + t;
            }
        }
    }
    for (int32_t h = 0; h < H; ++h) y_row[h] = oracle_f32_to_bf16(acc[h]);
    return 0;
}

int32_t oracle_combine(const oracle_cfg* c, const uint16_t* expert_out,
                       const int32_t* expert_ids, const int32_t* expand_idx,
                       const float* expert_scales, const int32_t* ep_recv_count,
                       const int64_t* recv_offsets, const uint8_t* mask,
                       const uint16_t* ori_x, uint16_t* y, float* acc)
{
    for (int32_t s = 0; s < c->W; ++s)
        for (int32_t i = 0; i < c->BS; ++i) {
            int32_t rc = oracle_combine_token(c, expert_out, expert_ids, expand_idx,
                                              expert_scales, ep_recv_count, recv_offsets,
                                              mask, ori_x, s, i, acc,
                                              y + ((size_t)s * c->BS + i) * c->H);
            if (rc != 0) return rc;
        }
    return 0;
}
