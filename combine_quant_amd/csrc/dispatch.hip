// dispatch.hip -- quantize each source token once and write it to its K packed rows.
//
// Vectorized path (H % 8 == 0, 16-byte aligned pointers): one workgroup per source token
// (s, i); each wavefront owns two slots of 64 16-byte vectors (8 bf16 elements per lane, so
// every load instruction covers 1 KiB of contiguous memory).  All waves issue their row
// loads first; threads 0..K-1 resolve the token's K destination rows meanwhile; one barrier
// publishes the rows (and, for mode 2, the per-wave maxima of the token).  Each wave then
// quantizes its slots in registers and stores them to the final row of every routed pick.
// Rows are read and written with the non-temporal cache policy (each is touched exactly
// once).  Small workgroups, many of them, keep every SIMD busy until the end of the launch.
//
// Destination rows follow the pages' placement rule (design doc §2.2.2 token reorder and
// §2.4 post-processing, merged into one address because every receiver lives in this GPU's
// memory): the (expert, source) segment base left in the workspace by the scan kernel plus
// the pick's expand_idx.
//
// Quantization (ops-transformer article, 功能说明 情形 2; low_latency_dispatch, 计算公式):
//   mode 0  rows copied bit for bit
//   mode 2  dyn = 127 / max|x_fp32| over the token (x_fp32 times the pick's expert smooth
//           row when smooth scales are given, which makes the work per pick), codes =
//           x_fp32 * dyn rounded half to even, scale = 1 / dyn
//   mode 4  per 32-element block: shared_exp = floor(log2 max|x|) - 8 (clamped at -127)
//   mode 5  per block: shared_exp = ceil(log2(max(max|x|, 1e-4) / 448))
//           codes = E4M3(x / 2^shared_exp); the stored scale is 2^shared_exp.
// In the vectorized path an MX block is 32 elements = 4 adjacent lanes of 8, reduced with two
// lane exchanges.
//
// The element-wise fallback (any H, any alignment) uses one workgroup per token with one
// element per lane (scatter_elem_kernel); an MX block is then 32 adjacent lanes.
#include "dc_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

// int8 code of one element: round half to even, saturate to +-127, NaN (0 * inf) -> 0.
__device__ __forceinline__ uint32_t int8_code(float f, float dyn)
{
    const float v = f * dyn;
    if (v != v) return 0u;
    const float r = fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
    return (uint32_t)(int32_t)r;
}

// Shared exponent of an MX block from the bit pattern of its absolute maximum.
template <int MODE>
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits)
{
    if (MODE == 4) {
        if (amax_bits == 0) return -127;
        const int ex = (int)(amax_bits >> 23);
        const int fl = ex != 0 ? ex - 127 : (31 - __clz(amax_bits)) - 149;   // floor(log2)
        return fl - 8 > -127 ? fl - 8 : -127;
    } else {
        const float c = fmaxf(__uint_as_float(amax_bits), 1e-4f);
        const uint32_t vb = __float_as_uint(c / 448.0f);                   // normal, > 0
        return (int)(vb >> 23) - 127 + ((vb & 0x7FFFFFu) != 0u ? 1 : 0);     // ceil(log2)
    }
}

// 2^e for e in [-127, 126] as a binary32 (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2f(int e)
{
    return e >= -126 ? __uint_as_float((uint32_t)(127 + e) << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------------------------------
// vectorized path: one workgroup per token, kTileSlots 64-vector slots per wave
// ---------------------------------------------------------------------------------------

constexpr int kTileSlots = 2;        // 64-vector slots (1 KiB of bf16 each) per wave
constexpr int kMaxTileWaves = 8;     // H <= 8192: at most 1024 vectors = 16 slots

__device__ __forceinline__ void unpack8(uint4 w, float (&f)[8])
{
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

__device__ __forceinline__ uint32_t absmax8(const float (&f)[8], uint32_t amax)
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t bits = __float_as_uint(f[c]) & 0x7FFFFFFFu;
        amax = amax > bits ? amax : bits;
    }
    return amax;
}

// Eight int8 codes of f * dyn for a finite dyn (dyn = 127 / amax with amax > 0 and not tiny):
// then |f * dyn| <= 127 * (1 + 2^-23), so no clamp is needed and no NaN can arise.  Adding
// 1.5 * 2^23 to the binary32 product puts the sum in [2^23, 2^24), where binary32 spacing is 1:
// the addition rounds the product to an integer, ties to even, and the low byte of the sum's
// bit pattern is that integer in two's complement.  Byte permutes gather the four low bytes.
__device__ __forceinline__ uint2 int8_codes8_finite(const float (&f)[8], float dyn)
{
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float v = f[q] * dyn;
        b[q] = __float_as_uint(v + 12582912.0f);
    }
    const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u),
                                              0x05040100u);
    const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u),
                                              0x05040100u);
    return make_uint2(lo, hi);
}

__device__ __forceinline__ uint2 pack_codes8(const uint32_t (&c)[8])
{
    return make_uint2((c[0] & 0xFF) | ((c[1] & 0xFF) << 8) | ((c[2] & 0xFF) << 16) | (c[3] << 24),
                      (c[4] & 0xFF) | ((c[5] & 0xFF) << 8) | ((c[6] & 0xFF) << 16) | (c[7] << 24));
}

template <int MODE, bool SMOOTH>
__global__ __launch_bounds__(kWave * kMaxTileWaves) void scatter_tile_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const int32_t* __restrict__ seg,
    const float* __restrict__ smooth, void* __restrict__ expand_x,
    float* __restrict__ dyn_scales, int32_t* __restrict__ assist, int W, int E, int BS,
    int H, int K, int ns, long long cap)
{
    __shared__ int32_t rows_lds[kMaxK];
    __shared__ int32_t exps_lds[kMaxK];
    __shared__ uint32_t red[2][kMaxTileWaves];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const long long tok = blockIdx.x;
    const int s = (int)(tok / BS);
    const int i = (int)(tok - (long long)s * BS);
    const int NV = H >> 3;

    // 1. this wave's slots of the token row, in flight before anything waits
    const uint4* xr = reinterpret_cast<const uint4*>(x) + tok * NV;
    uint4 raw[kTileSlots];
#pragma unroll
    for (int n = 0; n < kTileSlots; ++n) {
        const int v = lane + (wave * kTileSlots + n) * kWave;
        if (v < NV) raw[n] = load_stream(xr + v);
    }

    // 2. destination rows, resolved by threads 0..K-1
    if (threadIdx.x < K) {
        const long long p = tok * K + threadIdx.x;
        const int32_t ord = expand_idx[p];
        const int32_t e = ids[p];
        int32_t row = -1;
        if (ord >= 0 && e >= 0 && e < E) {
            const long long r = (long long)seg[(long long)e * W + s] + ord;
            if (r < cap) row = (int32_t)r;
        }
        rows_lds[threadIdx.x] = row;
        exps_lds[threadIdx.x] = e;
        if (row >= 0) {
            assist[(long long)row * 3 + 0] = s;
            assist[(long long)row * 3 + 1] = i;
            assist[(long long)row * 3 + 2] = threadIdx.x;
        }
    }

    // 3. the token's absolute maximum (mode 2 without smooth scales), per wave first
    if (MODE == 2 && !SMOOTH) {
        uint32_t amax = 0;
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = lane + (wave * kTileSlots + n) * kWave;
            if (v < NV) {
                float f[8];
                unpack8(raw[n], f);
                amax = absmax8(f, amax);
            }
        }
        amax = wave_max_u32(amax);
        if (lane == 0) red[0][wave] = amax;
    }
    __syncthreads();

    int rows[kMaxK];
    bool any = false;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        rows[k] = k < K ? __builtin_amdgcn_readfirstlane(rows_lds[k]) : -1;
        any |= rows[k] >= 0;
    }
    if (!any) return;                                      // uniform over the workgroup

    if (MODE == 0) {
        uint4* out = reinterpret_cast<uint4*>(expand_x);
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = lane + (wave * kTileSlots + n) * kWave;
            if (v >= NV) continue;
#pragma unroll
            for (int k = 0; k < kMaxK; ++k)
                if (rows[k] >= 0) store_stream(out + (long long)rows[k] * NV + v, raw[n]);
        }
        return;
    }

    uint2* out = reinterpret_cast<uint2*>(expand_x);     // 8 codes per vector

    if (MODE == 2 && !SMOOTH) {
        uint32_t amax = 0;
        for (int w = 0; w < nw; ++w) amax = amax > red[0][w] ? amax : red[0][w];
        const float dyn = 127.0f / __uint_as_float(amax);
        const bool finite = __float_as_uint(dyn) < 0x7F800000u;          // dyn > 0 here
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = lane + (wave * kTileSlots + n) * kWave;
            if (v >= NV) continue;
            float f[8];
            unpack8(raw[n], f);
            uint2 packed;
            if (finite) {
                packed = int8_codes8_finite(f, dyn);
            } else {
                uint32_t c[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) c[q] = int8_code(f[q], dyn);
                packed = pack_codes8(c);
            }
#pragma unroll
            for (int k = 0; k < kMaxK; ++k)
                if (rows[k] >= 0) store_stream(out + (long long)rows[k] * NV + v, packed);
        }
        if (threadIdx.x == 0) {
            const float scale = 1.0f / dyn;
#pragma unroll
            for (int k = 0; k < kMaxK; ++k)
                if (rows[k] >= 0) dyn_scales[rows[k]] = scale;
        }
        return;
    }

    if (MODE == 2) {   // smooth scales: one quantization per pick, on its expert's row
        // The picks run one after another (each needs a workgroup-wide maximum); the smooth
        // slice of the next routed pick is loaded into the other register buffer while the
        // current pick reduces, synchronizes and stores, so its latency is hidden.
        float4 sm_cur[kTileSlots][2], sm_nxt[kTileSlots][2];
        auto load_smooth = [&](int pick, float4 (&dst)[kTileSlots][2]) {
            const float4* sm =
                reinterpret_cast<const float4*>(smooth + (long long)exps_lds[pick] * H);
#pragma unroll
            for (int n = 0; n < kTileSlots; ++n) {
                const int v = lane + (wave * kTileSlots + n) * kWave;
                if (v < NV) {
                    dst[n][0] = sm[2 * v];
                    dst[n][1] = sm[2 * v + 1];
                }
            }
        };
        int pk = 0;
        while (pk < K && rows[pk] < 0) ++pk;                 // first routed pick (uniform)
        if (pk < K) load_smooth(pk, sm_cur);
        for (int round = 0; pk < K; ++round) {
            const int cur = round & 1;
            int nxt = pk + 1;
            while (nxt < K && rows[nxt] < 0) ++nxt;
            if (nxt < K) load_smooth(nxt, sm_nxt);
            const int prow = rows[pk];
            // x * smooth stays in registers between the maximum and the codes
            float f[kTileSlots][8];
            uint32_t amax = 0;
#pragma unroll
            for (int n = 0; n < kTileSlots; ++n) {
                const int v = lane + (wave * kTileSlots + n) * kWave;
                if (v < NV) {
                    unpack8(raw[n], f[n]);
                    const float4 a = sm_cur[n][0];
                    const float4 b = sm_cur[n][1];
                    f[n][0] = f[n][0] * a.x; f[n][1] = f[n][1] * a.y;
                    f[n][2] = f[n][2] * a.z; f[n][3] = f[n][3] * a.w;
                    f[n][4] = f[n][4] * b.x; f[n][5] = f[n][5] * b.y;
                    f[n][6] = f[n][6] * b.z; f[n][7] = f[n][7] * b.w;
                    amax = absmax8(f[n], amax);
                }
            }
            amax = wave_max_u32(amax);
            // alternating buffers: a wave can only write this buffer again two picks later,
            // after the next barrier, by which time every wave has read it
            if (lane == 0) red[cur][wave] = amax;
            __syncthreads();
            amax = 0;
            for (int w = 0; w < nw; ++w) amax = amax > red[cur][w] ? amax : red[cur][w];
            const float dyn = 127.0f / __uint_as_float(amax);
            const bool finite = __float_as_uint(dyn) < 0x7F800000u;
#pragma unroll
            for (int n = 0; n < kTileSlots; ++n) {
                const int v = lane + (wave * kTileSlots + n) * kWave;
                if (v >= NV) continue;
                uint2 packed;
                if (finite) {
                    packed = int8_codes8_finite(f[n], dyn);
                } else {
                    uint32_t c[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) c[q] = int8_code(f[n][q], dyn);
                    packed = pack_codes8(c);
                }
                store_stream(out + (long long)prow * NV + v, packed);
            }
            if (threadIdx.x == 0) dyn_scales[prow] = 1.0f / dyn;
#pragma unroll
            for (int n = 0; n < kTileSlots; ++n) {
                sm_cur[n][0] = sm_nxt[n][0];
                sm_cur[n][1] = sm_nxt[n][1];
            }
            pk = nxt;
        }
        return;
    }

    // MX modes 4 and 5: a 32-element block is 4 adjacent lanes of one wave
    const int nb = (H + kMxBlock - 1) / kMxBlock;
#pragma unroll
    for (int n = 0; n < kTileSlots; ++n) {
        const int v = lane + (wave * kTileSlots + n) * kWave;
        float f[8];
        uint32_t amax = 0;
        if (v < NV) {
            unpack8(raw[n], f);
            amax = absmax8(f, 0u);
        }
        amax = group_max_u32<4>(amax);
        if (v >= NV) continue;
        const int se = mx_shared_exp<MODE>(amax);
        const float inv = __uint_as_float((uint32_t)(127 - se) << 23);       // 2^-se, exact
        uint32_t c[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) c[q] = e4m3_code(f[q] * inv);
        const uint2 packed = pack_codes8(c);
        const bool lead = (v & 3) == 0;
        const float scale = pow2f(se);
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            if (rows[k] < 0) continue;
            store_stream(out + (long long)rows[k] * NV + v, packed);
            if (lead) dyn_scales[(long long)rows[k] * ns + (v >> 2)] = scale;
        }
    }
    if (threadIdx.x == 0 && ns > nb) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
            if (rows[k] >= 0) dyn_scales[(long long)rows[k] * ns + nb] = 0.0f;
    }
}

template <int MODE, bool SMOOTH>
hipError_t launch_tile_mode(const Shape& sh, const void* x, const int32_t* ids,
                            const int32_t* expand_idx, const int32_t* seg, const float* smooth,
                            void* expand_x, float* dyn_scales, int32_t* assist,
                            hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    const int slots = ((sh.H >> 3) + kWave - 1) / kWave;
    const int waves = (slots + kTileSlots - 1) / kTileSlots;        // <= kMaxTileWaves
    hipLaunchKernelGGL((scatter_tile_kernel<MODE, SMOOTH>), dim3((unsigned)T),
                       dim3(kWave * waves), 0, stream, static_cast<const uint16_t*>(x), ids,
                       expand_idx, seg, smooth, expand_x, dyn_scales, assist, sh.W, sh.E, sh.BS,
                       sh.H, sh.K, sh.scales_per_row, (long long)sh.cap);
    return hipGetLastError();
}

hipError_t launch_tile(const Shape& sh, const void* x, const int32_t* ids,
                       const int32_t* expand_idx, const int32_t* seg, const float* smooth,
                       void* expand_x, float* dyn_scales, int32_t* assist, hipStream_t stream)
{
    switch (sh.quant_mode) {
    case 0:
        return launch_tile_mode<0, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    case 2:
        if (smooth)
            return launch_tile_mode<2, true>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                             dyn_scales, assist, stream);
        return launch_tile_mode<2, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    case 4:
        return launch_tile_mode<4, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    case 5:
        return launch_tile_mode<5, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    default:
        return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------------------
// element-wise fallback: one workgroup per token, one element per lane
// ---------------------------------------------------------------------------------------

constexpr int kElemThreads = 1024;
constexpr int kElemPerLane = 8;      // H <= 8192 = 1024 lanes x 8

template <int MODE, bool SMOOTH>
__global__ __launch_bounds__(kElemThreads) void scatter_elem_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const int32_t* __restrict__ seg,
    const float* __restrict__ smooth, void* __restrict__ expand_x,
    float* __restrict__ dyn_scales, int32_t* __restrict__ assist, int W, int E, int BS,
    int H, int K, int ns, long long cap)
{
    __shared__ long long row_of[kMaxK];
    __shared__ int32_t exp_of[kMaxK];
    __shared__ uint32_t red[kElemThreads / kWave];

    const long long tok = blockIdx.x;
    const int s = (int)(tok / BS);
    const int i = (int)(tok - (long long)s * BS);
    const int t = threadIdx.x;
    const int nt = blockDim.x;

    if (t < K) {
        const int32_t ord = expand_idx[tok * K + t];
        const int32_t e = ids[tok * K + t];
        long long row = -1;
        if (ord >= 0 && e >= 0 && e < E) {
            row = (long long)seg[(long long)e * W + s] + ord;
            if (row >= cap) row = -1;
        }
        row_of[t] = row;
        exp_of[t] = e;
        if (row >= 0) {
            assist[row * 3 + 0] = s;
            assist[row * 3 + 1] = i;
            assist[row * 3 + 2] = t;
        }
    }
    __syncthreads();
    bool any = false;
    for (int k = 0; k < K; ++k) any |= row_of[k] >= 0;
    if (!any) return;

    const uint16_t* xr = x + tok * H;
    uint16_t raw[kElemPerLane];
#pragma unroll
    for (int n = 0; n < kElemPerLane; ++n) {
        const int h = t + n * nt;
        if (h < H) raw[n] = xr[h];
    }

    if (MODE == 0) {
        uint16_t* out = reinterpret_cast<uint16_t*>(expand_x);
        for (int k = 0; k < K; ++k) {
            const long long row = row_of[k];
            if (row < 0) continue;
#pragma unroll
            for (int n = 0; n < kElemPerLane; ++n) {
                const int h = t + n * nt;
                if (h < H) out[row * H + h] = raw[n];
            }
        }
        return;
    }

    uint8_t* out = reinterpret_cast<uint8_t*>(expand_x);

    if (MODE == 2) {
        // Without smooth scales every pick carries the same codes, so one pass serves all K;
        // with smooth scales each pick is quantized on its own expert's row.
        const int passes = SMOOTH ? K : 1;
        for (int pk = 0; pk < passes; ++pk) {
            if (SMOOTH && row_of[pk] < 0) continue;        // uniform over the workgroup
            const float* sm = SMOOTH ? smooth + (long long)exp_of[pk] * H : nullptr;
            uint32_t amax = 0;
#pragma unroll
            for (int n = 0; n < kElemPerLane; ++n) {
                const int h = t + n * nt;
                if (h < H) {
                    float f = bf16_lo(raw[n]);
                    if (SMOOTH) f = f * sm[h];
                    const uint32_t b = __float_as_uint(f) & 0x7FFFFFFFu;
                    amax = amax > b ? amax : b;
                }
            }
            amax = block_max_u32(amax, red);
            const float dyn = 127.0f / __uint_as_float(amax);
#pragma unroll
            for (int n = 0; n < kElemPerLane; ++n) {
                const int h = t + n * nt;
                if (h >= H) continue;
                float f = bf16_lo(raw[n]);
                if (SMOOTH) f = f * sm[h];
                const uint8_t c = (uint8_t)int8_code(f, dyn);
                if (SMOOTH) {
                    out[row_of[pk] * H + h] = c;
                } else {
                    for (int k = 0; k < K; ++k)
                        if (row_of[k] >= 0) out[row_of[k] * H + h] = c;
                }
            }
            if (t == 0) {
                const float scale = 1.0f / dyn;
                if (SMOOTH) {
                    dyn_scales[row_of[pk]] = scale;
                } else {
                    for (int k = 0; k < K; ++k)
                        if (row_of[k] >= 0) dyn_scales[row_of[k]] = scale;
                }
            }
        }
        return;
    }

    // MX modes 4 and 5: a 32-element block is 32 adjacent lanes
    const int nb = (H + kMxBlock - 1) / kMxBlock;
#pragma unroll
    for (int n = 0; n < kElemPerLane; ++n) {
        const int h = t + n * nt;
        if (n * nt >= H) break;                            // uniform across the workgroup
        float f = 0.0f;
        uint32_t amax = 0;
        if (h < H) {
            f = bf16_lo(raw[n]);
            amax = __float_as_uint(f) & 0x7FFFFFFFu;
        }
        amax = group_max_u32<kMxBlock>(amax);
        if (h >= H) continue;
        const int se = mx_shared_exp<MODE>(amax);
        const float inv = __uint_as_float((uint32_t)(127 - se) << 23);       // 2^-se, exact
        const uint8_t c = (uint8_t)e4m3_code(f * inv);
        const bool lead = (h % kMxBlock) == 0;
        const float scale = pow2f(se);
        for (int k = 0; k < K; ++k) {
            const long long row = row_of[k];
            if (row < 0) continue;
            out[row * H + h] = c;
            if (lead) dyn_scales[row * ns + h / kMxBlock] = scale;
        }
    }
    if (t == 0 && ns > nb) {
        for (int k = 0; k < K; ++k)
            if (row_of[k] >= 0) dyn_scales[row_of[k] * ns + nb] = 0.0f;
    }
}

template <int MODE, bool SMOOTH>
hipError_t launch_elem_mode(const Shape& sh, const void* x, const int32_t* ids,
                            const int32_t* expand_idx, const int32_t* seg, const float* smooth,
                            void* expand_x, float* dyn_scales, int32_t* assist,
                            hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    const int want = (sh.H + kWave - 1) / kWave * kWave;
    const int threads = want < kElemThreads ? want : kElemThreads;
    hipLaunchKernelGGL((scatter_elem_kernel<MODE, SMOOTH>), dim3((unsigned)T), dim3(threads),
                       0, stream, static_cast<const uint16_t*>(x), ids, expand_idx, seg, smooth,
                       expand_x, dyn_scales, assist, sh.W, sh.E, sh.BS, sh.H, sh.K,
                       sh.scales_per_row, (long long)sh.cap);
    return hipGetLastError();
}

hipError_t launch_elem(const Shape& sh, const void* x, const int32_t* ids,
                       const int32_t* expand_idx, const int32_t* seg, const float* smooth,
                       void* expand_x, float* dyn_scales, int32_t* assist, hipStream_t stream)
{
    switch (sh.quant_mode) {
    case 0:
        return launch_elem_mode<0, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    case 2:
        if (smooth)
            return launch_elem_mode<2, true>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                             dyn_scales, assist, stream);
        return launch_elem_mode<2, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    case 4:
        return launch_elem_mode<4, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    case 5:
        return launch_elem_mode<5, false>(sh, x, ids, expand_idx, seg, smooth, expand_x,
                                          dyn_scales, assist, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scatter(const Shape& sh, const void* x, const int32_t* expert_ids,
                          const int32_t* expand_idx, const int32_t* seg, const float* smooth,
                          void* expand_x, float* dynamic_scales, int32_t* assist_info,
                          bool vectorized, hipStream_t stream)
{
    if (vectorized)
        return launch_tile(sh, x, expert_ids, expand_idx, seg, smooth, expand_x,
                           dynamic_scales, assist_info, stream);
    return launch_elem(sh, x, expert_ids, expand_idx, seg, smooth, expand_x, dynamic_scales,
                       assist_info, stream);
}

}  // namespace moe_dc
