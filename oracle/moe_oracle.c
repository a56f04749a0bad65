/*
 * moe_oracle.c -- plain CPU oracle for MoE dispatch/combine (see moe_oracle.h for the pages).
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg; never by the product path.  Built with gcc -O2 -ffp-contract=off and no
 * fast-math, so every float operation below is one IEEE-754 binary32 operation rounded to
 * nearest-even, in the order written.
 *
 * Every function restates what the pages define, in the pages' order.  Where a page is
 * silent or garbled the reading taken is named inline (R1, R2, ...) and listed with its
 * reason in the design notes of the repository.
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

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits; largest finite 65504,
 * smallest normal 2^-14, subnormals m * 2^-24.  Widening is exact. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = h & 0x8000;
    int ex = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (ex == 0x1F) {
        if (m != 0) return NAN;
        return sign ? -INFINITY : INFINITY;
    }
    if (ex == 0) v = ldexp((double)m, -24);
    else v = ldexp(1.0 + m / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

/* Narrowing binary32 -> binary16, round to nearest, ties to even (the IEEE default); values
 * that round beyond 65504 become infinity; NaN stays NaN.  Same method as the fp8 encoders:
 * the binary16 spacing in the binade of |v| is 2^(floor(log2|v|) - 10), and 2^-24 all
 * through the subnormal range below 2^-14. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0x0000;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00);
    double a = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00);
    double quantum;
    if (a < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -24);
    } else {
        int ex;
        frexp(a, &ex);
        quantum = ldexp(1.0, (ex - 1) - 10);
    }
    double r = nearbyint(a / quantum) * quantum;
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00);      /* rounded past 65504 */
    uint16_t code;
    if (r < ldexp(1.0, -14)) {
        code = (uint16_t)(r / ldexp(1.0, -24));               /* 0..1024; 1024 = 2^-14 */
    } else {
        int ex;
        double m = frexp(r, &ex);
        int e2 = ex - 1;
        int mant = (int)((2.0 * m - 1.0) * 1024.0);            /* exact: 10 fraction bits */
        code = (uint16_t)(((e2 + 15) << 10) | mant);
    }
    return (uint16_t)(sign | code);
}

/* binary16 -> int8 (the second cast of the combine-side quantization chain float -> fp16 ->
 * int8): round half to even, saturate to [-127, 127], NaN -> 0 (readings R4, R5, R27). */
int8_t oracle_int8_from_f16(uint16_t h)
{
    return oracle_int8_from_f32(oracle_f16_to_f32(h));
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

/* OCP E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits, laid out like an IEEE binary
 * format: exponent field 31 holds the infinities (mantissa 0) and NaNs.  The largest finite
 * magnitude is 1.75 * 2^15 = 57344, the smallest normal 2^-14, and the subnormals are
 * m * 2^-16 for m = 1..3. */
float oracle_e5m2_to_f32(uint8_t code)
{
    int sign = code & 0x80;
    int ex = (code >> 2) & 0x1F;
    int m = code & 0x3;
    double v;
    if (ex == 0x1F) {
        if (m != 0) return NAN;
        return sign ? -INFINITY : INFINITY;
    }
    if (ex == 0) v = ldexp((double)m, -16);
    else v = ldexp(1.0 + m / 4.0, ex - 15);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest E5M2 value, ties to the even code.  Magnitudes at
 * or above 57344 saturate to 57344 (reading R6 again: a saturating cast, so no code is ever
 * infinite); NaN gives the NaN code; the sign is kept.  Same method as the E4M3 encoder:
 * the E5M2 spacing in the binade of |v| is 2^(floor(log2|v|) - 2), and 2^-16 all through
 * the subnormal range below 2^-14. */
uint8_t oracle_e5m2_from_f32(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 57344.0) return (uint8_t)(sign | 0x7B);
    double quantum;
    if (a < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -16);
    } else {
        int ex;
        frexp(a, &ex);               /* floor(log2 a) = ex - 1 */
        quantum = ldexp(1.0, (ex - 1) - 2);
    }
    double n = nearbyint(a / quantum);
    double r = n * quantum;          /* representable, <= 57344 because a < 57344 */
    uint8_t code;
    if (r < ldexp(1.0, -14)) {
        code = (uint8_t)(r / ldexp(1.0, -16));         /* 0..4; 4 is exactly 2^-14 = 0x04 */
    } else {
        int ex;
        double m = frexp(r, &ex);
        int e2 = ex - 1;
        int mant = (int)((2.0 * m - 1.0) * 4.0);       /* exact: 2m has 2 fraction bits */
        code = (uint8_t)(((e2 + 15) << 2) | mant);
    }
    return (uint8_t)(sign | code);
}

/* OCP E2M1 (fp4): 1 sign, 2 exponent (bias 1), 1 mantissa bit, no infinities or NaN.  The
 * eight magnitudes are 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4 and 6; a code is 4 bits. */
float oracle_e2m1_to_f32(uint8_t code)
{
    int sign = code & 0x8;
    int ex = (code >> 1) & 0x3;
    int m = code & 0x1;
    double v = ex == 0 ? 0.5 * m : ldexp(1.0 + m / 2.0, ex - 1);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest E2M1 value, ties to the even code, saturating
 * magnitudes >= 6 to 6 (reading R6 again; E2M1 has no NaN, so a NaN input is taken as a
 * contract violation and coded 6 with its sign, like any overflow).  Method of the fp8
 * encoders: spacing 2^(floor(log2|v|) - 1) in the binade of |v|, 0.5 below 1. */
uint8_t oracle_e2m1_from_f32(float v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs((double)v);
    if (isnan(v) || a >= 6.0) return (uint8_t)(sign | 0x7);
    double quantum;
    if (a < 1.0) {
        quantum = 0.5;
    } else {
        int ex;
        frexp(a, &ex);
        quantum = ldexp(1.0, (ex - 1) - 1);
    }
    double r = nearbyint(a / quantum) * quantum;     /* <= 6 because a < 6 */
    uint8_t code;
    if (r < 1.0) {
        code = (uint8_t)(r / 0.5);                    /* 0..2; 2 is exactly 1.0 = 0x2 */
    } else {
        int ex;
        double m = frexp(r, &ex);
        int e2 = ex - 1;
        int mant = (int)((2.0 * m - 1.0) * 2.0);      /* exact: 1 fraction bit */
        code = (uint8_t)(((e2 + 1) << 1) | mant);
    }
    return (uint8_t)(sign | code);
}

/* The int8 cast of every int8 mode (readings R4, R5; reading R22: the static mode 1 uses the
 * same cast): round half to even, saturate to [-127, 127], NaN -> 0. */
int8_t oracle_int8_from_f32(float v)
{
    if (isnan(v)) return 0;
    float r = nearbyintf(v);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* E8M0 byte of a power-of-two scale 2^e with e in [-127, 127]: the biased exponent e + 127
 * (the MX scale format; [SMP] 通信前量化 stores the MX shared-exponent scale as an E8M0 value
 * next to the fp8 codes).  frexpf handles the subnormal 2^-127 exactly: byte 0. */
uint8_t oracle_e8m0_from_scale(float s)
{
    int ex;
    frexpf(s, &ex);                  /* s = 0.5 * 2^ex */
    return (uint8_t)((ex - 1) + 127);
}

/* MX scales per row: one per 32-element block, padded to an even count (Align2 of
 * Ceil(H, 32)) as the dynamic_scales shape rule for quant modes 4/5 states ([LLD] 约束说明). */
int32_t oracle_mx_scale_count(int32_t H)
{
    int32_t nb = (H + 31) / 32;
    return nb + (nb & 1);
}

/* Element type of expand_x for a quant mode and a requested out_dtype (0 = the mode's
 * default).  [LLD] 约束说明 lists the allowed output types per mode: mode 0 keeps the input
 * type; mode 1 int8; mode 2 int8, E4M3 or E5M2; mode 3 E4M3 or E5M2; modes 4/5 E4M3 or
 * E5M2, modes 4/5 also E2M1 (the hifloat8 and E1M2 types there are not covered).  -1 for any
 * other pairing. */
int32_t oracle_code_type(int32_t quant_mode, int32_t out_dtype)
{
    switch (quant_mode) {
    case 0:
        return out_dtype == 0 ? ORACLE_CODE_BF16 : -1;
    case 1:
        return (out_dtype == 0 || out_dtype == ORACLE_CODE_INT8) ? ORACLE_CODE_INT8 : -1;
    case 2:
        if (out_dtype == 0) return ORACLE_CODE_INT8;
        return (out_dtype == ORACLE_CODE_INT8 || out_dtype == ORACLE_CODE_E4M3 ||
                out_dtype == ORACLE_CODE_E5M2) ? out_dtype : -1;
    case 3:
        if (out_dtype == 0) return ORACLE_CODE_E4M3;
        return (out_dtype == ORACLE_CODE_E4M3 || out_dtype == ORACLE_CODE_E5M2) ? out_dtype
                                                                                : -1;
    case 4:
    case 5:
        if (out_dtype == 0) return ORACLE_CODE_E4M3;
        return (out_dtype == ORACLE_CODE_E4M3 || out_dtype == ORACLE_CODE_E5M2 ||
                out_dtype == ORACLE_CODE_E2M1) ? out_dtype : -1;
    default:
        return -1;
    }
}

/* Bytes of one expand_x row: 2H for bf16, H/2 for E2M1 (two codes per byte, the element of
 * even index in the low nibble: reading R31), else H. */
int32_t oracle_code_row_bytes(int32_t code_type, int32_t H)
{
    if (code_type == ORACLE_CODE_BF16) return 2 * H;
    if (code_type == ORACLE_CODE_E2M1) return H / 2;
    return H;
}

/* Scales per expand_x row ([LLD] 约束说明, dynamic_scales shapes): none for modes 0 and 1,
 * one for mode 2, Ceil(H, 128) for mode 3, Align2(Ceil(H, 32)) for modes 4/5. */
int32_t oracle_scale_count(int32_t quant_mode, int32_t H)
{
    switch (quant_mode) {
    case 2: return 1;
    case 3: return (H + 127) / 128;
    case 4:
    case 5: return oracle_mx_scale_count(H);
    default: return 0;
    }
}

/* ------------------------------------------------------------------------------------- */
/* quantization                                                                          */
/* ------------------------------------------------------------------------------------- */

/* Largest finite magnitude of a code type: the dst_type_max of the dynamic formulas and the
 * fp8_max of the clip variant. */
static float code_max(int32_t ct)
{
    switch (ct) {
    case ORACLE_CODE_INT8: return 127.0f;
    case ORACLE_CODE_E4M3: return 448.0f;
    case ORACLE_CODE_E5M2: return 57344.0f;
    default: return 6.0f;                            /* E2M1 */
    }
}

/* emax of an MX element type: the exponent of its largest power of two (E4M3 2^8 = 256,
 * E5M2 2^15, E2M1 2^2 = 4), used by the MX shared exponent. */
static int code_emax(int32_t ct)
{
    return ct == ORACLE_CODE_E4M3 ? 8 : ct == ORACLE_CODE_E5M2 ? 15 : 2;
}

static uint8_t encode(int32_t ct, float v)
{
    if (ct == ORACLE_CODE_INT8) return (uint8_t)oracle_int8_from_f32(v);
    if (ct == ORACLE_CODE_E4M3) return oracle_e4m3_from_f32(v);
    if (ct == ORACLE_CODE_E5M2) return oracle_e5m2_from_f32(v);
    return oracle_e2m1_from_f32(v);
}

/* One dynamic-scale segment [h0, h1) of the fp32 row f ([LLD] 计算公式, quant_mode 2 over the
 * whole token and quant_mode 3 over each group; [OPS] 功能说明 情形 2):
 *   dyn   = dst_type_max / max|f| over the segment
 *   q     = Cast(f * dyn, dst type)
 *   scale = 1.0 / dyn
 * An all-zero segment gives dyn = +inf and products 0 * inf = NaN; every NaN product is
 * encoded as 0 (reading R21: R5 taken for the fp8 types too), and its scale is 1/inf = 0. */
/* Token elements (x, ori_x, expert outputs, y): bf16 (token_dtype 0) or IEEE binary16 (1).
 * Widening is exact for both; narrowing rounds to nearest, ties to even. */
static float tok_to_f32(int32_t token_dtype, uint16_t b)
{
    return token_dtype ? oracle_f16_to_f32(b) : oracle_bf16_to_f32(b);
}

static uint16_t f32_to_tok(int32_t token_dtype, float f)
{
    return token_dtype ? oracle_f32_to_f16(f) : oracle_f32_to_bf16(f);
}

static float quant_dynamic(int32_t ct, const float* f, int32_t h0, int32_t h1, uint8_t* q)
{
    float amax = 0.0f;
    for (int32_t h = h0; h < h1; ++h)
        if (fabsf(f[h]) > amax) amax = fabsf(f[h]);
    float dyn = code_max(ct) / amax;
    for (int32_t h = h0; h < h1; ++h) {
        float v = f[h] * dyn;
        q[h] = isnan(v) ? 0 : encode(ct, v);
    }
    return 1.0f / dyn;
}

/* floor(log2(a)) for a finite a > 0, exactly: frexpf gives a = m * 2^ex with m in [0.5,1). */
static int ilog2_floor(float a)
{
    int ex;
    frexpf(a, &ex);
    return ex - 1;
}

/* One MX block [h0, h1) (32 elements, the last one may be short).
 * quant_mode 4 ([LLD] 计算公式, quant_mode=4; [OPS] 接口级量化模式扩展):
 *   shared_exp = floor(log2(max|x| over the block)) - emax   (emax 8 for E4M3, 15 for E5M2)
 *   q = Cast(x / 2^shared_exp, fp8)
 * Reading R7: max(x) is the block's absolute maximum.  Reading R8: an all-zero block takes
 * shared_exp = -127, and shared_exp is clamped below at -127 (the E8M0 range).
 * quant_mode 5, the clip variant ([LLD] 计算公式, quant_mode=5):
 *   max_abs_clamp = max(max|x|, 1e-4);  shared_exp = ceil(log2(max_abs_clamp / fp8_max))
 *   q = CastToFp8(x / 2^shared_exp)     (fp8_max 448 for E4M3, 57344 for E5M2)
 * Reading R9: max_abs_clamp / fp8_max is one fp32 division and its ceil(log2) is exact.
 * Reading R10: the block's scale is 2^shared_exp, the dequant multiplier (codes * scale ~ x). */
static float quant_mx_block(int32_t ct, int32_t clip, const float* f, int32_t h0, int32_t h1,
                            uint8_t* q)
{
    float amax = 0.0f;
    for (int32_t h = h0; h < h1; ++h)
        if (fabsf(f[h]) > amax) amax = fabsf(f[h]);
    int se;
    if (!clip) {
        if (amax == 0.0f) se = -127;
        else se = ilog2_floor(amax) - code_emax(ct);
        if (se < -127) se = -127;
    } else {
        float c = amax > 1e-4f ? amax : 1e-4f;
        float v = c / code_max(ct);
        int ex;
        float m = frexpf(v, &ex);    /* v = m * 2^ex; v is a power of two iff m == 0.5 */
        se = (m == 0.5f) ? ex - 1 : ex;
    }
    float sc = ldexpf(1.0f, se);     /* 2^-127 is a binary32 subnormal: exact */
    for (int32_t h = h0; h < h1; ++h) q[h] = encode(ct, f[h] / sc);
    return sc;
}

/* Quantize one token row x (bf16 [H]; binary16 through oracle_quant_row_tok) for a quant mode and code type, after multiplying it
 * by `pre` when given: pre_len 1 = one scalar for every element, pre_len H = one value per
 * element, 0 = no multiplier ([LLD] 计算公式: x_fp32 = CastToFp32(x) * scales; the scales
 * tensor may be a scalar, a row shared by the experts or the routed expert's row, per
 * 约束说明 of modes 1-3; reading R23: modes 2 and 3 take the same three shapes as mode 1).
 *   mode 1: q = Cast(x_fp32, int8) with the static scales already applied; no scales out
 *   mode 2: one dynamic segment over the whole row; one scale
 *   mode 3: dynamic segments of 128 elements (the last may be short); Ceil(H,128) scales
 *           (reading R20: the group length is the 128 of the scale shape (A, Ceil(H,128)))
 *   mode 4/5: MX blocks of 32; Align2(Ceil(H,32)) scales, the pad entry 0
 * codes: oracle_code_row_bytes bytes (int8 two's complement, fp8 codes, or E2M1 codes two per
 * byte).  Returns 0, or -1 when the code type, the multiplier or the mode do not go together. */
int32_t oracle_quant_row(int32_t quant_mode, int32_t code_type, const uint16_t* x,
                         const float* pre, int32_t pre_len, int32_t H, void* codes,
                         float* scales)
{
    return oracle_quant_row_tok(0, quant_mode, code_type, x, pre, pre_len, H, codes, scales);
}

int32_t oracle_quant_row_tok(int32_t token_dtype, int32_t quant_mode, int32_t code_type,
                             const uint16_t* x, const float* pre, int32_t pre_len, int32_t H,
                             void* codes, float* scales)
{
    if (quant_mode < 1 || quant_mode > 5) return -1;
    if (oracle_code_type(quant_mode, code_type) != code_type) return -1;
    if (code_type == ORACLE_CODE_E2M1 && H % 2 != 0) return -1;   /* [LLD]: H even for fp4 */
    if (pre_len != 0 && pre_len != 1 && pre_len != H) return -1;
    if ((pre_len != 0) != (pre != NULL)) return -1;
    if (quant_mode >= 4 && pre_len != 0) return -1;
    if (quant_mode == 1 && pre_len == 0) return -1;
    uint8_t* q = (uint8_t*)codes;
    float* f = (float*)malloc((size_t)H * sizeof(float));
    for (int32_t h = 0; h < H; ++h) {
        f[h] = tok_to_f32(token_dtype, x[h]);
        if (pre_len == 1) f[h] = f[h] * pre[0];
        else if (pre_len == H) f[h] = f[h] * pre[h];
    }
    if (quant_mode == 1) {
        for (int32_t h = 0; h < H; ++h) q[h] = encode(code_type, f[h]);
    } else if (quant_mode == 2) {
        scales[0] = quant_dynamic(code_type, f, 0, H, q);
    } else if (quant_mode == 3) {
        for (int32_t g = 0; g * 128 < H; ++g) {
            int32_t h1 = g * 128 + 128 < H ? g * 128 + 128 : H;
            scales[g] = quant_dynamic(code_type, f, g * 128, h1, q);
        }
    } else {
        /* E2M1 codes are made one per byte first, then packed two per byte (R31) */
        uint8_t* one = code_type == ORACLE_CODE_E2M1 ? (uint8_t*)malloc((size_t)H) : q;
        int32_t nb = (H + 31) / 32;
        for (int32_t b = 0; b < nb; ++b) {
            int32_t h1 = b * 32 + 32 < H ? b * 32 + 32 : H;
            scales[b] = quant_mx_block(code_type, quant_mode == 5, f, b * 32, h1, one);
        }
        for (int32_t b = nb; b < oracle_mx_scale_count(H); ++b) scales[b] = 0.0f;
        if (code_type == ORACLE_CODE_E2M1) {
            for (int32_t h = 0; h < H; h += 2) q[h / 2] = (uint8_t)(one[h] | (one[h + 1] << 4));
            free(one);
        }
    }
    free(f);
    return 0;
}

/* Per-token dynamic int8 quantization, quant_mode 2 ([OPS] 功能说明 情形 2; [LLD] 计算公式,
 * quant_mode=2): dyn = 127 / max|x_fp32|, q = CastToInt8(x_fp32 * dyn), scale = 1.0 / dyn,
 * with x_fp32 the token times the smooth-scale row when one is given. */
void oracle_quant_int8_row(const uint16_t* x, const float* smooth_or_null, int32_t H,
                           int8_t* q, float* scale)
{
    oracle_quant_row(2, ORACLE_CODE_INT8, x, smooth_or_null, smooth_or_null ? H : 0, H, q,
                     scale);
}

/* MX E4M3 quantization of one row (quant_mode 4, or 5 when clip is set). */
void oracle_quant_mx_row(const uint16_t* x, int32_t H, int32_t clip, uint8_t* codes,
                         float* scales)
{
    oracle_quant_row(clip ? 5 : 4, ORACLE_CODE_E4M3, x, NULL, 0, H, codes, scales);
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
 *   mode 0 ([LLD] quant_mode=0): the token row (bf16 or binary16) is moved unchanged; no scales.
 *   modes 1-5: the row quantized by oracle_quant_row for the configured code type.  The
 *   scales tensor ([LLD] 约束说明, modes 1-3) is a scalar (scales_kind 1), a row shared by
 *   every expert (2) or the routed expert's row of an [E][H] table (3); with kind 3 the
 *   quantization is per pair.
 *   expand_x [cap][row bytes] (bf16 patterns for mode 0; E2M1 two codes per byte; else bytes);
 *   dynamic_scales [cap][scale count] fp32, or bytes when scale_format is 1: each MX scale
 *   2^e as its E8M0 byte e + 127 ([SMP] 通信前量化), pad bytes 0 (reading R24); with
 *   scale_format 2 each MX scale is the formula's literal transmitted value 1.0 / 2^e (one fp32
 *   division, exact for a power of two), pad 0;
 *   assist_info [cap][3].
 * Returns -2 for a mode / code type / scales kind / scale format that do not go together,
 * -3 when the scales pointer disagrees with scales_kind, -1 for an out-of-range id. */
int32_t oracle_dispatch(const oracle_cfg* c, const uint16_t* x, const int32_t* expert_ids,
                        const float* scales_or_null, const uint8_t* mask, void* expand_x,
                        void* dynamic_scales, int32_t* expand_idx, int32_t* assist_info,
                        int32_t* ep_recv_count, int64_t* expert_token_nums,
                        int64_t* recv_offsets, int32_t* cnt_scratch)
{
    const int32_t H = c->H, mode = c->quant_mode;
    const int32_t ct = oracle_code_type(mode, c->out_dtype);
    if (ct < 0) return -2;
    if (c->scales_kind < 0 || c->scales_kind > 3) return -2;
    if ((mode == 0 || mode >= 4) && c->scales_kind != 0) return -2;
    if (mode == 1 && c->scales_kind == 0) return -2;
    if (c->scale_format != 0 && !((c->scale_format == 1 || c->scale_format == 2) && mode >= 4))
        return -2;
    if ((c->scales_kind != 0) != (scales_or_null != NULL)) return -3;
    if (oracle_route(c, expert_ids, mask, cnt_scratch, expand_idx) != 0) return -1;
    oracle_recv_counts(c, cnt_scratch, ep_recv_count, expert_token_nums, recv_offsets);
    const int32_t ns = oracle_scale_count(mode, H);
    const int32_t nb = (H + 31) / 32;
    const size_t row_bytes = (size_t)oracle_code_row_bytes(ct, H);
    if (ct == ORACLE_CODE_E2M1 && H % 2 != 0) return -2;
    float* rowsc = (float*)malloc((size_t)(ns > 0 ? ns : 1) * sizeof(float));
    for (int32_t s = 0; s < c->W; ++s)
        for (int32_t i = 0; i < c->BS; ++i)
            for (int32_t k = 0; k < c->K; ++k) {
                size_t p = ((size_t)s * c->BS + i) * c->K + k;
                int32_t ord = expand_idx[p];
                if (ord < 0) continue;
                int32_t e = expert_ids[p];
                int64_t row = oracle_dest_row(c, ep_recv_count, recv_offsets, s, e, ord);
                const uint16_t* xr = x + ((size_t)s * c->BS + i) * H;
                if (mode == 0) {
                    memcpy((uint16_t*)expand_x + (size_t)row * H, xr, (size_t)H * 2);
                } else {
                    const float* pre = NULL;
                    int32_t pre_len = 0;
                    if (c->scales_kind == 1) { pre = scales_or_null; pre_len = 1; }
                    if (c->scales_kind == 2) { pre = scales_or_null; pre_len = H; }
                    if (c->scales_kind == 3) { pre = scales_or_null + (size_t)e * H; pre_len = H; }
                    oracle_quant_row_tok(c->token_dtype, mode, ct, xr, pre, pre_len, H,
                                         (uint8_t*)expand_x + (size_t)row * row_bytes, rowsc);
                    for (int32_t b = 0; b < ns; ++b) {
                        if (c->scale_format == 1)
                            ((uint8_t*)dynamic_scales)[(size_t)row * ns + b] =
                                b < nb ? oracle_e8m0_from_scale(rowsc[b]) : 0;
                        else if (c->scale_format == 2)   /* [LLD] 计算公式: 1.0 / dynamic_scales_value */
                            ((float*)dynamic_scales)[(size_t)row * ns + b] =
                                b < nb ? 1.0f / rowsc[b] : 0.0f;
                        else
                            ((float*)dynamic_scales)[(size_t)row * ns + b] = rowsc[b];
                    }
                }
                assist_info[(size_t)row * 3 + 0] = s;
                assist_info[(size_t)row * 3 + 1] = i;
                assist_info[(size_t)row * 3 + 2] = k;
            }
    free(rowsc);
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
 * to the token type (bf16 or binary16).  A token with no active pick therefore gives +0. */
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
                float t = w * tok_to_f32(c->token_dtype, src[h]);
                acc[h] = acc[h] + t;
            }
        } else if (e < zero_end) {
            continue;
        } else {
            if (ori_x == NULL) return -1;
            const uint16_t* src = ori_x + ((size_t)s * c->BS + i) * H;
            for (int32_t h = 0; h < H; ++h) {
                float t = w * tok_to_f32(c->token_dtype, src[h]);
                acc[h] = acc[h] + t;
            }
        }
    }
    for (int32_t h = 0; h < H; ++h) y_row[h] = f32_to_tok(c->token_dtype, acc[h]);
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

/* ------------------------------------------------------------------------------------- */
/* combine-side int8 block quantization ([SMP] 通信前量化, Combine 的 INT8 block 量化)       */
/* ------------------------------------------------------------------------------------- */

/* Blocks of 8 elements: the page processes 32-byte blocks of 8 floats (reading R26), so a
 * row has Ceil(H, 8) blocks, the last one short when 8 does not divide H. */
int32_t oracle_combine_block_count(int32_t H)
{
    return (H + 7) / 8;
}

/* Expert-side quantization of one expert-output row, in the page's order: widen to float;
 * per block: absolute maximum (Abs, BlockReduceMax); scale = amax * (1 / 127) (Muls by the
 * reciprocal of SCALE_PARAM = 127.0, the reciprocal one fp32 division); q = x / scale (Div);
 * then the casts float -> fp16 -> int8 (reading R27: each cast rounds to nearest even; the
 * int8 cast saturates at +-127 and maps NaN to 0, so an all-zero block, 0 / 0, gives codes
 * 0 with scale 0). */
void oracle_combine_quant_row(const uint16_t* row, int32_t H, int8_t* q, float* scales)
{
    oracle_combine_quant_row_tok(0, row, H, q, scales);
}

void oracle_combine_quant_row_tok(int32_t token_dtype, const uint16_t* row, int32_t H, int8_t* q,
                                  float* scales)
{
    const float inv127 = 1.0f / 127.0f;
    for (int32_t b = 0; b * 8 < H; ++b) {
        int32_t h0 = b * 8;
        int32_t h1 = h0 + 8 < H ? h0 + 8 : H;
        float amax = 0.0f;
        for (int32_t h = h0; h < h1; ++h) {
            float a = fabsf(tok_to_f32(token_dtype, row[h]));
            if (a > amax) amax = a;
        }
        float scale = amax * inv127;
        for (int32_t h = h0; h < h1; ++h) {
            float v = tok_to_f32(token_dtype, row[h]) / scale;
            q[h] = oracle_int8_from_f16(oracle_f32_to_f16(v));
        }
        scales[b] = scale;
    }
}

/* Source-side dequantization: int8 -> fp16 -> float (both exact), times the block's scale
 * (one fp32 multiply). */
void oracle_combine_dequant_row(const int8_t* q, const float* scales, int32_t H, float* out)
{
    for (int32_t h = 0; h < H; ++h) {
        float v = oracle_f16_to_f32(oracle_f32_to_f16((float)q[h]));
        out[h] = v * scales[h / 8];
    }
}

/* Every packed expert-output row [0, recv_offsets[W]) quantized; codes [cap][H] int8,
 * scales [cap][Ceil(H, 8)] fp32.  Rows past recv_offsets[W] are not touched. */
int32_t oracle_combine_quantize(const oracle_cfg* c, const uint16_t* expert_out,
                                const int64_t* recv_offsets, int8_t* codes, float* scales)
{
    const int32_t H = c->H, nb = oracle_combine_block_count(H);
    for (int64_t r = 0; r < recv_offsets[c->W]; ++r)
        oracle_combine_quant_row_tok(c->token_dtype, expert_out + (size_t)r * H, H,
                                     codes + (size_t)r * H, scales + (size_t)r * nb);
    return 0;
}

int32_t oracle_combine_int8_token(const oracle_cfg* c, const int8_t* codes, const float* scales,
                                  const int32_t* expert_ids, const int32_t* expand_idx,
                                  const float* expert_scales, const int32_t* ep_recv_count,
                                  const int64_t* recv_offsets, const uint8_t* mask,
                                  const uint16_t* ori_x, int32_t s, int32_t i, float* acc,
                                  float* rowbuf, uint16_t* y_row)
{
    const int32_t H = c->H, nb = oracle_combine_block_count(H);
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
            oracle_combine_dequant_row(codes + (size_t)row * H, scales + (size_t)row * nb, H,
                                       rowbuf);
            for (int32_t h = 0; h < H; ++h) {
                float t = w * rowbuf[h];
                acc[h] = acc[h] + t;
            }
        } else if (e >= zero_end) {
            if (ori_x == NULL) return -1;
            const uint16_t* src = ori_x + ((size_t)s * c->BS + i) * H;
            for (int32_t h = 0; h < H; ++h) {
                float t = w * tok_to_f32(c->token_dtype, src[h]);
                acc[h] = acc[h] + t;
            }
        }
    }
    for (int32_t h = 0; h < H; ++h) y_row[h] = f32_to_tok(c->token_dtype, acc[h]);
    return 0;
}

/* The combine of oracle_combine_token with each routed pick's row dequantized first: the
 * same addressing ([DDD] §3.4.2), the same fp32 sum in k order of w * row, zero experts
 * adding nothing and copy experts adding w * ori_x (reading R28: ori_x stays on its source
 * rank, so it is never quantized); the result rounded to the token type.  Token by token through
 * oracle_combine_int8_token. */
int32_t oracle_combine_int8(const oracle_cfg* c, const int8_t* codes, const float* scales,
                            const int32_t* expert_ids, const int32_t* expand_idx,
                            const float* expert_scales, const int32_t* ep_recv_count,
                            const int64_t* recv_offsets, const uint8_t* mask,
                            const uint16_t* ori_x, uint16_t* y, float* acc, float* rowbuf)
{
    for (int32_t s = 0; s < c->W; ++s)
        for (int32_t i = 0; i < c->BS; ++i) {
            int32_t rc = oracle_combine_int8_token(c, codes, scales, expert_ids, expand_idx,
                                                   expert_scales, ep_recv_count, recv_offsets,
                                                   mask, ori_x, s, i, acc, rowbuf,
                                                   y + ((size_t)s * c->BS + i) * c->H);
            if (rc != 0) return rc;
        }
    return 0;
}

/* ------------------------------------------------------------------------------------- */
/* weights with the rows, and the scatter-back combine                                   */
/* ------------------------------------------------------------------------------------- */

/* Each dispatched row's pick weight, row-aligned with expand_x: the weight travels with the
 * token ([OPS] 参数说明, expand_scales_out: the weights of the tokens this card outputs).  The
 * row's pick is read from its source triple (s, i, k) in assist_info.  Rows at or past
 * recv_offsets[W] are not written. */
int32_t oracle_expand_scales(const oracle_cfg* c, const int32_t* assist_info,
                             const int64_t* recv_offsets, const float* expert_scales,
                             float* expand_scales)
{
    for (int64_t r = 0; r < recv_offsets[c->W]; ++r) {
        int32_t s = assist_info[r * 3 + 0], i = assist_info[r * 3 + 1], k = assist_info[r * 3 + 2];
        if (s < 0 || s >= c->W || i < 0 || i >= c->BS || k < 0 || k >= c->K) return -1;
        expand_scales[r] = expert_scales[((size_t)s * c->BS + i) * c->K + k];
    }
    return 0;
}

/* The sample's scatter-back combine ([SMP] Combine 功能介绍 计算步骤 and 源码实现), in its
 * order.  First every expert-side row r in [0, recv_offsets[W]) is sent back to its source:
 * its triple (s, i, k) = assist_info[r] gives the slot epOffset = i * K + k of rank s's
 * receive window, and the row is copied there.  Then each source token waits for its K
 * slots and sums them in pick order, each times its expert scale (the source's own
 * expert_scales, reading R30), in fp32; the shared expert's output, when given, is added
 * after the K picks (reading R29); the sum is rounded to the token type.
 * Picks that were never dispatched (inactive, special experts) have no slot: a zero expert
 * or an inactive pick adds nothing, a copy expert adds w * ori_x, as in oracle_combine.
 *   window_scratch [W][BS*K][H] bf16; acc_scratch [H] fp32. */
int32_t oracle_combine_scatter(const oracle_cfg* c, const uint16_t* expert_out,
                               const int32_t* assist_info, const int64_t* recv_offsets,
                               const int32_t* expert_ids, const float* expert_scales,
                               const uint8_t* mask, const uint16_t* ori_x,
                               const uint16_t* shared_x, uint16_t* y, uint16_t* window,
                               float* acc)
{
    const int32_t H = c->H, K = c->K;
    const int32_t zero_end = c->E + c->zero_expert_num;
    const int32_t copy_end = zero_end + c->copy_expert_num;
    memset(window, 0, (size_t)c->W * c->BS * K * H * sizeof(uint16_t));
    for (int64_t r = 0; r < recv_offsets[c->W]; ++r) {
        int32_t s = assist_info[r * 3 + 0], i = assist_info[r * 3 + 1], k = assist_info[r * 3 + 2];
        if (s < 0 || s >= c->W || i < 0 || i >= c->BS || k < 0 || k >= K) return -1;
        size_t ep_offset = (size_t)i * K + k;
        memcpy(window + ((size_t)s * c->BS * K + ep_offset) * H, expert_out + (size_t)r * H,
               (size_t)H * sizeof(uint16_t));
    }
    for (int32_t s = 0; s < c->W; ++s)
        for (int32_t i = 0; i < c->BS; ++i) {
            for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                size_t p = ((size_t)s * c->BS + i) * K + k;
                if (!pair_active(c, mask, s, i, k)) continue;
                int32_t e = expert_ids[p];
                float w = expert_scales[p];
                if (e < 0 || e >= copy_end) return -1;
                const uint16_t* src;
                if (e < c->E) src = window + ((size_t)s * c->BS * K + (size_t)i * K + k) * H;
                else if (e < zero_end) continue;
                else if (ori_x == NULL) return -1;
                else src = ori_x + ((size_t)s * c->BS + i) * H;
                for (int32_t h = 0; h < H; ++h) {
                    float t = w * tok_to_f32(c->token_dtype, src[h]);
                    acc[h] = acc[h] + t;
                }
            }
            if (shared_x) {
                const uint16_t* sh = shared_x + ((size_t)s * c->BS + i) * H;
                for (int32_t h = 0; h < H; ++h) acc[h] = acc[h] + tok_to_f32(c->token_dtype, sh[h]);
            }
            uint16_t* yr = y + ((size_t)s * c->BS + i) * H;
            for (int32_t h = 0; h < H; ++h) yr[h] = f32_to_tok(c->token_dtype, acc[h]);
        }
    return 0;
}
