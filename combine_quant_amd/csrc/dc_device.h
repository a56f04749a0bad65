// dc_device.h -- device helpers for the gfx950 dispatch/combine kernels.
//
// Everything here is written for CDNA4 wave64 execution.  Numerics follow the formulas of
// the pages exactly as the library header states them: one binary32 operation per written
// float operation (the library is built with -ffp-contract=off, so no FMA fusion), IEEE
// division, subnormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_dc {

constexpr int kWave = 64;
constexpr int kMaxK = 16;          // largest top-k the pages allow
constexpr int kMxBlock = 32;       // MX block length (elements sharing one exponent)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 bit pattern, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// IEEE binary16 token elements: widening is exact; narrowing is the hardware conversion,
// which rounds to nearest even (overflow to infinity, subnormals kept, NaN stays NaN).
__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return f32_to_f16(lo) | (f32_to_f16(hi) << 16);
}

// Token elements (x, ori_x, shared_x, expert outputs, y) of either type: F16 selects binary16,
// else bf16.
template <bool F16>
__device__ __forceinline__ float tok_lo(uint32_t w) { return F16 ? f16_lo(w) : bf16_lo(w); }
template <bool F16>
__device__ __forceinline__ float tok_hi(uint32_t w) { return F16 ? f16_hi(w) : bf16_hi(w); }
template <bool F16>
__device__ __forceinline__ uint32_t pack_tok2(float lo, float hi)
{
    return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}
__device__ __forceinline__ float tok_lo_rt(uint32_t w, bool f16)
{
    return f16 ? f16_lo(w) : bf16_lo(w);
}
__device__ __forceinline__ uint32_t f32_to_tok_rt(float f, bool f16)
{
    return f16 ? f32_to_f16(f) : f32_to_bf16_rne(f);
}

// E4M3 ("fn" variant: bias 7, no infinities, 448 largest) code of a finite binary32 value:
// nearest, ties to even, magnitudes >= 448 saturate to 448, sign kept (also on zero).
// Normal results: round the binary32 significand to 3 fraction bits at bit 20 and rebias
// the exponent from 127 to 7.  Below 2^-6 the E4M3 grid is uniform with step 2^-9, so the
// code is |v| * 2^9 rounded to an integer (8 lands exactly on the smallest normal, 0x08).
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E00000u) return sign | 0x7Eu;                 // |v| >= 448
    if (a < 0x3C800000u) {                                     // |v| < 2^-6
        const float scaled = __uint_as_float(a) * 512.0f;      // exact power-of-two scaling
        return sign | (uint32_t)__builtin_rintf(scaled);
    }
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// E5M2 (bias 15, largest finite 57344) code of a finite binary32 value: nearest, ties to
// even, magnitudes >= 57344 saturate to 57344 (never the infinity code), sign kept.  Normal
// results round the significand to 2 fraction bits at bit 21 and rebias from 127 to 15;
// below 2^-14 the grid is uniform with step 2^-16.  A value below 57344 cannot round past
// it, since 57344 itself is on the grid.
__device__ __forceinline__ uint32_t e5m2_code(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x47600000u) return sign | 0x7Bu;                 // |v| >= 57344
    if (a < 0x38800000u) {                                     // |v| < 2^-14
        const float scaled = __uint_as_float(a) * 65536.0f;    // exact power-of-two scaling
        return sign | (uint32_t)__builtin_rintf(scaled);
    }
    const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
    return sign | ((((r >> 23) - 112u) << 2) | ((r >> 21) & 3u));
}

// E2M1 (fp4: bias 1, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) 4-bit code of a finite binary32
// value: nearest, ties to even, magnitudes >= 6 saturate to 6, sign in bit 3.  Below 1 the
// grid is 0, 0.5, 1 (step 0.5: the code is |v| * 2 rounded); above, the significand is rounded
// to 1 fraction bit at bit 22 and the exponent rebiased from 127 to 1.
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 28) & 0x8u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x40C00000u) return sign | 0x7u;                  // |v| >= 6
    if (a < 0x3F800000u)                                       // |v| < 1
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
    const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
    return sign | ((((r >> 23) - 126u) << 1) | ((r >> 22) & 1u));
}

// Streaming (non-temporal) 16- and 8-byte global accesses, for rows that are touched once.
// They lower to global loads/stores with the non-temporal cache policy, which keeps the
// once-read / once-written rows from displacing reusable lines in L2 and the Infinity Cache.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(uint4* p, uint4 o)
{
    const u32x4_t v = {o.x, o.y, o.z, o.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ void store_stream(uint2* p, uint2 o)
{
    const u32x2_t v = {o.x, o.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

// Buffer resource over the `bytes` bytes at `base` (a wave-uniform address).  Accesses
// through it are range-checked by the hardware: a load past the end returns 0 and a store
// past it is dropped.  Code that covers a ragged row end this way needs no branch around the
// access, so the compiler can count outstanding memory operations exactly and wait only for
// the ones a value depends on.  Every access here is 16, 8 or 4 bytes at a multiple of its
// size, so it lies either wholly inside or wholly past the end.
constexpr int32_t kRsrcWord3 = 0x00020000;       // gfx9 family: 32-bit data format, no swizzle
constexpr uint32_t kRsrcPastEnd = 0x80000000u;    // an offset past the end of every resource
constexpr int kRsrcNonTemporal = 2;              // aux bits: the nt cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// `off` is the lane's whole byte offset, passed as the vector offset (the compiler may move
// a constant part into the instruction's immediate offset, which the range check includes);
// the scalar offset operand stays 0, since it is not part of the range check.
__device__ __forceinline__ float4 rsrc_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

__device__ __forceinline__ void rsrc_store_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 o)
{
    const u32x2_t v = {o.x, o.y};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kRsrcNonTemporal);
}

__device__ __forceinline__ void rsrc_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float o)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), r, (int)off, 0, 0);
}

// Value of `v` in lane `lane` (a compile-time or wave-uniform index), for every lane.
__device__ __forceinline__ int lane_value(int v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Largest value across the 64 lanes of a wave (unsigned), in every lane: the device
// library's wave reduction (DPP row operations, then two lane reads).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return __ockl_wfred_max_u32(v);
}

// DPP lane patterns (GFX9 encodings) used by group_max_u32; every lane of a row of 16 reads a
// valid lane, so no bound control is involved.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i within each half row of 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15 - i within each row of 16

__device__ __forceinline__ uint32_t dpp_max(uint32_t v, uint32_t o) { return v > o ? v : o; }

// Largest value over groups of G adjacent lanes (G a power of two <= 64), in every lane of
// the group.  Within a row of 16 lanes the exchanges are DPP moves (ALU latency); beyond, lane
// shuffles.  After the quad steps all four lanes of a quad hold its maximum, so mirroring the
// half row pairs each quad with its neighbour, and mirroring the row pairs the two halves.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v)
{
    if (G >= 2)
        v = dpp_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, false));
    if (G >= 4)
        v = dpp_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, false));
    if (G >= 8)
        v = dpp_max(v,
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowHalfMirror, 0xF, 0xF, false));
    if (G >= 16)
        v = dpp_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowMirror, 0xF, 0xF, false));
#pragma unroll
    for (int off = 16; off < G; off <<= 1) v = dpp_max(v, __shfl_xor(v, off, kWave));
    return v;
}

// Block-wide unsigned max; `scratch` holds one word per wave.  Every thread gets the result.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* scratch)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = (blockDim.x + kWave - 1) / kWave;
    v = wave_max_u32(v);
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int w = 0; w < nwaves; ++w) r = r > scratch[w] ? r : scratch[w];
    __syncthreads();
    return r;
}

}  // namespace moe_dc
