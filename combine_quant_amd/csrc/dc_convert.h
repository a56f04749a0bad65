// dc_convert.h -- the conversions of the dispatch kernels that use gfx950 instructions in
// place of bit-level code: static int8, fp8 and fp4 element codes, and a short correctly
// rounded division.
// Each is exact only where an exhaustive check over every binary32 input says so;
// selfcheck.hip runs those checks on the GPU against the bit-level encoders of dc_device.h and
// the correctly rounded division.
#pragma once
#include "dc_device.h"
#include "dc_internal.h"

namespace moe_dc {

// int8 code of one value: round half to even, saturate to +-127, NaN -> 0 (the two's complement
// byte is the code).
__device__ __forceinline__ uint32_t int8_code(float v)
{
    if (v != v) return 0u;
    const float r = fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
    return (uint32_t)(int32_t)r;
}

// Eight int8 codes of v as int8_code gives them, packed element 0 lowest: a NaN becomes 0, one
// med3 clamps to +-127, and adding 1.5 * 2^23 puts the value in [2^23, 2^24), where binary32
// spacing is 1, so the addition rounds it to an integer (ties to even) whose two's complement is
// the low byte of the sum's bit pattern; byte permutes gather the eight low bytes.
__device__ __forceinline__ uint2 static_int8_codes8(const float (&v)[8])
{
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float c = v[q] != v[q] ? 0.0f : __builtin_amdgcn_fmed3f(v[q], -127.0f, 127.0f);
        b[q] = __float_as_uint(c + 12582912.0f);
    }
    const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u),
                                              0x05040100u);
    const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u),
                                              0x05040100u);
    return make_uint2(lo, hi);
}

// Eight E4M3 or E5M2 codes of finite or infinite values, by the conversion instructions of
// gfx950 (two values per instruction).  They round to nearest, ties to even, keep the sign of
// zero and give the subnormal codes, exactly as e4m3_code / e5m2_code do -- checked on the GPU
// against those encoders for every finite binary32 value -- but past the largest finite value
// they give the NaN code, so each value is first clamped to +-type_max (one med3), where the
// software codes saturate.  A NaN input is not allowed (med3 would turn it into -type_max).
template <int CT>
__device__ __forceinline__ uint2 fp8_codes8_hw(const float (&v)[8])
{
    constexpr float m = CT == kCodeE4m3 ? 448.0f : 57344.0f;
    float c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) c[q] = __builtin_amdgcn_fmed3f(v[q], -m, m);
    uint32_t lo, hi;
    if (CT == kCodeE4m3) {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], (int)hi, true);
    } else {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[4], c[5], 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[6], c[7], (int)hi, true);
    }
    return make_uint2(lo, hi);
}

// Eight E2M1 codes of finite or infinite values as one word, element 0 in the lowest nibble,
// by gfx950's scaled fp4 conversion with scale 1 (two values per instruction, one byte each).
// After a clamp to +-6 it gives e2m1_code's code for every finite binary32 value (checked on
// the GPU); a NaN input is not allowed.
__device__ __forceinline__ uint32_t fp4_word_hw(const float (&v)[8])
{
    float c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) c[q] = __builtin_amdgcn_fmed3f(v[q], -6.0f, 6.0f);
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, c[0], c[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[2], c[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[4], c[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[6], c[7], 1.0f, 3);
    return w;
}

// a / b, correctly rounded, for a constant a > 0 and any b >= 0 (zero, infinite and NaN
// included): where b's exponent field lies in [LO, 252], a reciprocal estimate and two fused
// multiply-adds; elsewhere the correctly rounded division.  An exhaustive GPU check over every
// binary32 b found the short sequence equal to the correctly rounded quotient for a = 448 with
// exponent fields 8..252, a = 57344 with 15..252 and a = 1 with 1..252, and not outside those
// ranges (tiny b, whose quotient overflows, and huge b); a caller passes the LO checked for
// its a, and moe_dc_selfcheck_conversions re-checks each pairing used.
template <int LO>
__device__ __forceinline__ float div_rn(float a, float b)
{
    const uint32_t ex = __float_as_uint(b) >> 23;
    if (ex >= (uint32_t)LO && ex <= 252u) {
        const float y = __builtin_amdgcn_rcpf(b);
        const float q0 = a * y;
        const float r = __builtin_fmaf(-q0, b, a);
        return __builtin_fmaf(r, y, q0);
    }
    return a / b;
}

}  // namespace moe_dc
