// combine.hip -- top-K weighted gather back to the source tokens.
//
// One workgroup per source token.  Lanes 0..K-1 first resolve each pick's source row with
// the design doc's addressing rule (§3.4.2: the owner rank's window + the expert's offset
// inside it + expand_idx), written here with the dispatch outputs: recv_offsets[r] + the
// running total of ep_recv_count just before (local expert j, source s) + expand_idx.
// Special experts follow the low_latency_dispatch formulas: a zero expert contributes
// nothing, a copy expert contributes its weight times ori_x.
//
// Each lane then owns 16-byte column vectors of the token; for each it issues the K row
// loads first (all in flight together) and only then accumulates in pick order, one fp32
// multiply and one fp32 add per pick (the sample article's combine: weight each expert row,
// accumulate in fp32, cast down), and stores the bf16 rounding of the sum.
//
// Vectorized path (H % 8 == 0, 16-byte aligned): a token's row is cut into chunks of 128
// 16-byte vectors, each handled by one independent wavefront, which resolves
// the token's sources in lanes 0..K-1 and broadcasts them as wave-uniform values; expert rows
// are read and y is written with the non-temporal policy; no workgroup barrier.  Element-wise
// fallback (any H, any alignment): one workgroup per token, one element per lane.
//
// Combine-side int8 block quantization (the sample article's combine INT8 block
// quantization, 通信前量化): the expert side compresses each expert-output row into int8
// codes with one fp32 scale per 8 elements (scale = amax * (1/127), code = int8(fp16(x /
// scale)), each cast rounding to nearest even); the combine then reads codes and scales
// instead of bf16 rows and dequantizes each element (int8 -> fp16 -> float is exact, times
// the scale) before weighting it.  One 8-element block is exactly one lane's vector, so the
// block maximum needs no lane exchange, and a lane reads 12 bytes per pick instead of 16.
#include "dc_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

constexpr int kNone = -1;   // inactive pick, zero expert, or unresolvable
constexpr int kCopy = -2;   // copy expert: read ori_x

// Source of pick k of token tok: its expert_out row (>= 0), kCopy for a copy expert, or
// kNone.  With INV = false the row follows the design doc's addressing (§3.4.2: the owner
// rank's window + the expert's offset inside it + expand_idx), written with the dispatch
// outputs: recv_offsets[r] + the running total of ep_recv_count just before (local expert
// j, source s) + expand_idx.  With INV = true, `pick_rows` is the map written by the
// scatter-back step (slot tok * K + k -> the row that was sent back to it).  Rows outside
// [0, cap) are treated as unresolvable.
// The loads that depend only on the pick (expert id, expand_idx or slot row, mask byte) are
// issued together, then the two that depend on the expert (the rank's window start and the
// running total), so a task waits two load round trips before its row loads, not one per
// field.
template <bool INV>
__device__ __forceinline__ int pick_source(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ pick_rows,
    const int32_t* __restrict__ ep_recv_count, const int64_t* __restrict__ recv_offsets,
    const uint8_t* __restrict__ mask, int mask_kind, int W, int E, int L, int K, int zero_end,
    int id_end, long long cap, long long tok, int s, int k)
{
    const long long p = tok * K + k;
    const int32_t e = ids[p];
    const int32_t ord = pick_rows[p];
    const bool on = mask_kind == 0 || mask[mask_kind == 1 ? tok : p] != 0;
    if (!on || e < 0) return kNone;
    if (e < E && INV) return (ord >= 0 && ord < cap) ? (int)ord : kNone;
    if (e < E) {
        if (ord < 0) return kNone;
        const int r = e / L;
        const int j = e - r * L;
        const long long flat = (long long)j * W + s;
        const long long window = recv_offsets[r];
        const long long base =
            flat == 0 ? 0 : (long long)ep_recv_count[(long long)r * L * W + flat - 1];
        const long long row = window + base + ord;
        return (row >= 0 && row < cap) ? (int)row : kNone;
    }
    return (e >= zero_end && e < id_end) ? kCopy : kNone;
}

// acc[c] = acc[c] + w * element c of eight token values (bf16, or binary16 with F16; one
// multiply, one add each)
template <bool F16>
__device__ __forceinline__ void accumulate8(uint4 v, float w, float (&acc)[8])
{
    const float f[8] = {tok_lo<F16>(v.x), tok_hi<F16>(v.x), tok_lo<F16>(v.y), tok_hi<F16>(v.y),
                        tok_lo<F16>(v.z), tok_hi<F16>(v.z), tok_lo<F16>(v.w), tok_hi<F16>(v.w)};
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = acc[c] + w * f[c];
}

// Element c (0..3) of four int8 codes packed in a word, as a float (exact).
__device__ __forceinline__ float code_at(uint32_t w, int c)
{
    return (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * c));
}

// acc[c] = acc[c] + w * (code_c * scale): dequantize eight int8 codes of one block (one
// multiply), then weight and accumulate (one multiply, one add)
__device__ __forceinline__ void accumulate8_int8(uint2 q, float scale, float w, float (&acc)[8])
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float t0 = code_at(q.x, c) * scale;
        acc[c] = acc[c] + w * t0;
        const float t1 = code_at(q.y, c) * scale;
        acc[4 + c] = acc[4 + c] + w * t1;
    }
}

typedef uint32_t u32x2_ld_t __attribute__((ext_vector_type(2)));

// Non-temporal 16-byte load through a pointer marked as global memory: a row base picked
// among several buffers at run time would otherwise be accessed with flat instructions.
typedef const __attribute__((address_space(1))) u32x4_t* global_u32x4_ptr;

typedef const __attribute__((address_space(1))) u32x2_ld_t* global_u32x2_ptr;
typedef const __attribute__((address_space(1))) float* global_f32_ptr;

__device__ __forceinline__ uint4 load_row(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load((global_u32x4_ptr)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 load_row8(const uint2* p)
{
    const u32x2_ld_t v = __builtin_nontemporal_load((global_u32x2_ptr)p);
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float load_row4(const float* p)
{
    return __builtin_nontemporal_load((global_f32_ptr)p);
}

__device__ __forceinline__ uint2 load_stream8(const uint2* p)
{
    const u32x2_ld_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_ld_t*>(p));
    return make_uint2(v.x, v.y);
}

constexpr int kWavesPerBlock = 4;

// 64-vector slots of one token per wave task: two, so a lane has 2K row loads in flight
// (at K = 16 that halves the waves per SIMD, and is still faster than one slot).
constexpr int slots_per_task(int) { return 2; }

// One wave task = one token x SLOTS slots of 64 16-byte vectors.  A token's row is
// split across several independent waves (each resolves the token's K sources itself), so a
// launch is many short tasks: the hardware keeps every SIMD busy to the end instead of
// leaving a long, thinly occupied last round of whole-token waves.
// Q = 0: bf16 expert rows.  Q = 1: int8 codes [cap][H] and fp32 block scales [cap][H/8]
// (qscales), one block per lane vector; a routed pick's buffer entry then holds the two code
// words and the scale's bits.
// INV selects the scatter-back addressing (expand_idx then holds the slot -> row map) and
// SHARED adds the shared expert's bf16 output after the K picks.
template <int KMAX, int SLOTS, int Q, bool INV, bool SHARED, bool F16>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void combine_wave_kernel(
    const void* __restrict__ expert_out, const float* __restrict__ qscales,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ expand_idx,
    const float* __restrict__ weights, const int32_t* __restrict__ ep_recv_count,
    const int64_t* __restrict__ recv_offsets, const uint8_t* __restrict__ mask, int mask_kind,
    const uint16_t* __restrict__ ori_x, const uint16_t* __restrict__ shared_x,
    uint16_t* __restrict__ y, int W, int E, int L, int BS, int H, int K, int zero_end,
    int id_end, long long cap, long long T, int tasks_per_token)
{
    const int lane = threadIdx.x & (kWave - 1);
    // the wave's index, as a wave-uniform value (so the task's row bases stay scalar)
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const long long task = (long long)blockIdx.x * kWavesPerBlock + wave;
    const long long tok = task / tasks_per_token;
    if (tok >= T) return;                                  // whole wave
    const int slot0 = (int)(task - tok * tasks_per_token) * SLOTS;
    const int s = (int)(tok / BS);
    const int NV = H >> 3;

    int src = kNone;
    float wk = 0.0f;
    if (lane < K) {
        wk = weights[tok * K + lane];
        src = pick_source<INV>(ids, expand_idx, ep_recv_count, recv_offsets, mask, mask_kind,
                               W, E, L, K, zero_end, id_end, cap, tok, s, lane);
    }
    int srcs[KMAX];
    float ws[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        srcs[k] = k < K ? lane_value(src, k) : kNone;
        ws[k] = lane_value(wk, k);
    }

    // One load per pick and slot from a wave-uniform base: the pick's expert-output row, or
    // ori_x for a copy expert (bf16 rows).  The K loads of a slot then go out back to back;
    // loading alternatives into the same registers on two paths would make the compiler
    // wait for every earlier load before each of them.
    const uint4* eo = reinterpret_cast<const uint4*>(expert_out);
    const uint2* eq = reinterpret_cast<const uint2*>(expert_out);
    // ori_x is only read for copy experts, which exist only when it is given
    const uint4* self = reinterpret_cast<const uint4*>(ori_x ? ori_x : y) + tok * NV;
    uint4* yr = reinterpret_cast<uint4*>(y) + tok * NV;
    const uint4* rowp[KMAX];       // valid where `loads` has bit k
    uint32_t loads = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        rowp[k] = eo;
        if (srcs[k] >= 0) {
            rowp[k] = eo + (long long)srcs[k] * NV;
            loads |= 1u << k;
        } else if (Q == 0 && srcs[k] == kCopy) {
            rowp[k] = self;
            loads |= 1u << k;
        }
    }
    uint4 buf[SLOTS][KMAX];
    uint4 shv[SLOTS];
#pragma unroll
    for (int n = 0; n < SLOTS; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v < NV) {
            if (SHARED) shv[n] = load_stream(reinterpret_cast<const uint4*>(shared_x) + tok * NV + v);
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (!(loads & (1u << k))) continue;
                if (Q == 0) {
                    buf[n][k] = load_row(rowp[k] + v);
                } else {
                    const long long r = srcs[k];               // a routed pick's row
                    const uint2 q = load_row8(eq + r * NV + v);
                    const float sc = load_row4(qscales + r * NV + v);
                    buf[n][k] = make_uint4(q.x, q.y, __float_as_uint(sc), 0u);
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < SLOTS; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v < NV) {
            float acc[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (srcs[k] == kNone) continue;
                if (Q == 1 && srcs[k] >= 0)
                    accumulate8_int8(make_uint2(buf[n][k].x, buf[n][k].y),
                                     __uint_as_float(buf[n][k].z), ws[k], acc);
                else if (Q == 1)                    // copy expert: its ori_x vector, read here
                    accumulate8<F16>(self[v], ws[k], acc);
                else
                    accumulate8<F16>(buf[n][k], ws[k], acc);
            }
            if (SHARED) accumulate8<F16>(shv[n], 1.0f, acc);   // 1 * a token value is exact
            store_stream(yr + v,
                         make_uint4(pack_tok2<F16>(acc[0], acc[1]), pack_tok2<F16>(acc[2], acc[3]),
                                    pack_tok2<F16>(acc[4], acc[5]), pack_tok2<F16>(acc[6], acc[7])));
        }
    }
}

// Int8 combine with 16-element lanes (H % 16 == 0): per pick a lane reads one 16-byte code
// vector and one 8-byte pair of block scales (two blocks) instead of 8 + 4 bytes, so every
// load instruction moves twice the bytes.  One wave task = one token x 64 lanes x 16
// elements.  A copy expert's ori_x half-rows are read when they are accumulated.
template <int KMAX, bool F16>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void combine_int8_wide_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ qscales,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ expand_idx,
    const float* __restrict__ weights, const int32_t* __restrict__ ep_recv_count,
    const int64_t* __restrict__ recv_offsets, const uint8_t* __restrict__ mask, int mask_kind,
    const uint16_t* __restrict__ ori_x, uint16_t* __restrict__ y, int W, int E, int L, int BS,
    int H, int K, int zero_end, int id_end, long long cap, long long T, int tasks_per_token)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long long task = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const long long tok = task / tasks_per_token;
    if (tok >= T) return;                                  // whole wave
    const int u = lane + (int)(task - tok * tasks_per_token) * kWave;
    const int s = (int)(tok / BS);
    const int NU = H >> 4;                                 // 16-element units per row
    const int NV = H >> 3;

    int src = kNone;
    float wk = 0.0f;
    if (lane < K) {
        wk = weights[tok * K + lane];
        src = pick_source<false>(ids, expand_idx, ep_recv_count, recv_offsets, mask, mask_kind,
                               W, E, L, K, zero_end, id_end, cap, tok, s, lane);
    }
    int srcs[KMAX];
    float ws[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        srcs[k] = k < K ? lane_value(src, k) : kNone;
        ws[k] = lane_value(wk, k);
    }
    // lanes past the row's last unit still take part in the lane exchange before the stores
    const bool live = u < NU;

    const uint4* cq = reinterpret_cast<const uint4*>(codes);
    const uint2* sq = reinterpret_cast<const uint2*>(qscales);
    const uint4* self = ori_x ? reinterpret_cast<const uint4*>(ori_x) + tok * NV : nullptr;
    uint4 cbuf[KMAX];
    uint2 sbuf[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (live && srcs[k] >= 0) {
            cbuf[k] = load_stream(cq + (long long)srcs[k] * NU + u);
            sbuf[k] = load_stream8(sq + (long long)srcs[k] * NU + u);
        }
    }
    float lo[8], hi[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        lo[c] = 0.0f;
        hi[c] = 0.0f;
    }
    if (live) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (srcs[k] >= 0) {
                accumulate8_int8(make_uint2(cbuf[k].x, cbuf[k].y), __uint_as_float(sbuf[k].x),
                                 ws[k], lo);
                accumulate8_int8(make_uint2(cbuf[k].z, cbuf[k].w), __uint_as_float(sbuf[k].y),
                                 ws[k], hi);
            } else if (srcs[k] == kCopy) {
                accumulate8<F16>(self[2 * u], ws[k], lo);
                accumulate8<F16>(self[2 * u + 1], ws[k], hi);
            }
        }
    }
    // Lane l holds output vectors 2u and 2u + 1 (u = u0 + l).  Stored as they are, each store
    // instruction would cover every other 16 bytes of the wave's 2 KiB; instead lane j
    // writes vector 2u0 + j, then 2u0 + 64 + j, taken from lane j / 2 (resp. 32 + j / 2) --
    // its first vector when j is even, its second when j is odd -- so each store instruction
    // covers 1 KiB contiguously.
    const uint4 va = make_uint4(pack_tok2<F16>(lo[0], lo[1]), pack_tok2<F16>(lo[2], lo[3]),
                                pack_tok2<F16>(lo[4], lo[5]), pack_tok2<F16>(lo[6], lo[7]));
    const uint4 vb = make_uint4(pack_tok2<F16>(hi[0], hi[1]), pack_tok2<F16>(hi[2], hi[3]),
                                pack_tok2<F16>(hi[4], hi[5]), pack_tok2<F16>(hi[6], hi[7]));
    const bool odd = (lane & 1) != 0;
    const int v0 = 2 * (u - lane);                         // the wave's first output vector
    uint4* yr = reinterpret_cast<uint4*>(y) + tok * NV;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int from = h * (kWave / 2) + (lane >> 1);
        const uint32_t ax = __shfl(va.x, from, kWave), bx = __shfl(vb.x, from, kWave);
        const uint32_t ay = __shfl(va.y, from, kWave), by = __shfl(vb.y, from, kWave);
        const uint32_t az = __shfl(va.z, from, kWave), bz = __shfl(vb.z, from, kWave);
        const uint32_t aw = __shfl(va.w, from, kWave), bw = __shfl(vb.w, from, kWave);
        const int v = v0 + h * kWave + lane;
        if (v < NV)
            store_stream(yr + v, odd ? make_uint4(bx, by, bz, bw) : make_uint4(ax, ay, az, aw));
    }
}

template <int KMAX>
hipError_t launch_int8_wide_k(const Shape& sh, const int8_t* codes, const float* qscales,
                              const int32_t* ids, const int32_t* expand_idx, const float* w,
                              const int32_t* erc, const int64_t* roff, const uint8_t* mask,
                              const void* ori_x, void* y, hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    const int tasks_per_token = ((sh.H >> 4) + kWave - 1) / kWave;
    const long long tasks = T * tasks_per_token;
    const unsigned blocks = (unsigned)((tasks + kWavesPerBlock - 1) / kWavesPerBlock);
#define MOE_DC_INT8_WIDE(F)                                                                 \
    hipLaunchKernelGGL((combine_int8_wide_kernel<KMAX, F>), dim3(blocks),                   \
                       dim3(kWave * kWavesPerBlock), 0, stream, codes, qscales, ids,        \
                       expand_idx, w, erc, roff, mask, sh.mask_kind,                        \
                       static_cast<const uint16_t*>(ori_x), static_cast<uint16_t*>(y), sh.W, \
                       sh.E, sh.L, sh.BS, sh.H, sh.K, sh.zero_end, sh.id_end,               \
                       (long long)sh.cap, T, tasks_per_token)
    if (sh.tok_f16) MOE_DC_INT8_WIDE(true);
    else MOE_DC_INT8_WIDE(false);
#undef MOE_DC_INT8_WIDE
    return hipGetLastError();
}

template <int KMAX, int Q, bool INV, bool SHARED>
hipError_t launch_wave_k(const Shape& sh, const void* expert_out, const float* qscales,
                         const int32_t* ids, const int32_t* expand_idx, const float* w,
                         const int32_t* erc, const int64_t* roff, const uint8_t* mask,
                         const void* ori_x, const void* shared_x, void* y, hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    const int slots = ((sh.H >> 3) + kWave - 1) / kWave;
    constexpr int kSlots = slots_per_task(KMAX);
    const int tasks_per_token = (slots + kSlots - 1) / kSlots;
    const long long tasks = T * tasks_per_token;
    const unsigned blocks = (unsigned)((tasks + kWavesPerBlock - 1) / kWavesPerBlock);
#define MOE_DC_WAVE(F)                                                                      \
    hipLaunchKernelGGL((combine_wave_kernel<KMAX, kSlots, Q, INV, SHARED, F>), dim3(blocks), \
                       dim3(kWave * kWavesPerBlock), 0, stream, expert_out, qscales, ids,   \
                       expand_idx, w, erc, roff, mask, sh.mask_kind,                        \
                       static_cast<const uint16_t*>(ori_x),                                 \
                       static_cast<const uint16_t*>(shared_x), static_cast<uint16_t*>(y),   \
                       sh.W, sh.E, sh.L, sh.BS, sh.H, sh.K, sh.zero_end, sh.id_end,         \
                       (long long)sh.cap, T, tasks_per_token)
    if (sh.tok_f16) MOE_DC_WAVE(true);
    else MOE_DC_WAVE(false);
#undef MOE_DC_WAVE
    return hipGetLastError();
}

template <int Q, bool INV, bool SHARED>
hipError_t launch_wave(const Shape& sh, const void* eo, const float* qs, const int32_t* ids,
                       const int32_t* ei, const float* w, const int32_t* erc,
                       const int64_t* roff, const uint8_t* mask, const void* ori_x,
                       const void* shared_x, void* y, hipStream_t stream)
{
#define MOE_DC_ARGS sh, eo, qs, ids, ei, w, erc, roff, mask, ori_x, shared_x, y, stream
    if (sh.K <= 2) return launch_wave_k<2, Q, INV, SHARED>(MOE_DC_ARGS);
    if (sh.K <= 4) return launch_wave_k<4, Q, INV, SHARED>(MOE_DC_ARGS);
    if (sh.K <= 8) return launch_wave_k<8, Q, INV, SHARED>(MOE_DC_ARGS);
    return launch_wave_k<16, Q, INV, SHARED>(MOE_DC_ARGS);
#undef MOE_DC_ARGS
}

constexpr int kElemThreads = 1024;
constexpr int kElemPerLane = 8;      // H <= 8192 = 1024 lanes x 8

// Element-wise combine; Q as for combine_wave_kernel (codes [cap][H], scales [cap][Ceil(H,8)]).
template <int KMAX, int Q, bool INV>
__global__ __launch_bounds__(kElemThreads) void combine_elem_kernel(
    const void* __restrict__ expert_out, const float* __restrict__ qscales,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ expand_idx,
    const float* __restrict__ weights, const int32_t* __restrict__ ep_recv_count,
    const int64_t* __restrict__ recv_offsets, const uint8_t* __restrict__ mask, int mask_kind,
    const uint16_t* __restrict__ ori_x, const uint16_t* __restrict__ shared_x,
    uint16_t* __restrict__ y, int W, int E, int L, int BS, int H, int K, int zero_end,
    int id_end, long long cap, int tok_f16)
{
    __shared__ int src_of[KMAX];
    __shared__ float w_of[KMAX];
    const long long tok = blockIdx.x;
    const int s = (int)(tok / BS);
    const int t = threadIdx.x;
    const int nb = (H + 7) / 8;
    if (t < K) {
        src_of[t] = pick_source<INV>(ids, expand_idx, ep_recv_count, recv_offsets, mask,
                                     mask_kind, W, E, L, K, zero_end, id_end, cap, tok, s, t);
        w_of[t] = weights[tok * K + t];
    }
    __syncthreads();
    const uint16_t* eo = static_cast<const uint16_t*>(expert_out);
    const int8_t* eq = static_cast<const int8_t*>(expert_out);
    const uint16_t* self = ori_x ? ori_x + tok * H : nullptr;
    uint16_t* yr = y + tok * H;
#pragma unroll 1
    for (int n = 0; n < kElemPerLane; ++n) {
        const int h = t + n * blockDim.x;
        if (h >= H) break;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int src = src_of[k];
            if (src == kNone) continue;
            float v;
            if (src >= 0 && Q == 1) {
                const float t0 = (float)eq[(long long)src * H + h];
                v = t0 * qscales[(long long)src * nb + h / 8];
            } else {
                v = tok_lo_rt(src >= 0 ? eo[(long long)src * H + h] : self[h], tok_f16 != 0);
            }
            acc = acc + w_of[k] * v;
        }
        if (shared_x) acc = acc + tok_lo_rt(shared_x[tok * H + h], tok_f16 != 0);
        yr[h] = (uint16_t)f32_to_tok_rt(acc, tok_f16 != 0);
    }
}

template <int KMAX, int Q, bool INV>
hipError_t launch_elem_k(const Shape& sh, const void* expert_out, const float* qscales,
                         const int32_t* ids, const int32_t* expand_idx, const float* w,
                         const int32_t* erc, const int64_t* roff, const uint8_t* mask,
                         const void* ori_x, const void* shared_x, void* y, hipStream_t stream)
{
    const int want = (sh.H + kWave - 1) / kWave * kWave;
    const int threads = want < kElemThreads ? want : kElemThreads;
    const long long T = (long long)sh.W * sh.BS;
    hipLaunchKernelGGL((combine_elem_kernel<KMAX, Q, INV>), dim3((unsigned)T), dim3(threads),
                       0, stream, expert_out, qscales, ids, expand_idx, w, erc, roff, mask,
                       sh.mask_kind, static_cast<const uint16_t*>(ori_x),
                       static_cast<const uint16_t*>(shared_x), static_cast<uint16_t*>(y),
                       sh.W, sh.E, sh.L, sh.BS, sh.H, sh.K, sh.zero_end, sh.id_end,
                       (long long)sh.cap, sh.tok_f16);
    return hipGetLastError();
}

template <int Q, bool INV>
hipError_t launch_elem(const Shape& sh, const void* eo, const float* qs, const int32_t* ids,
                       const int32_t* ei, const float* w, const int32_t* erc,
                       const int64_t* roff, const uint8_t* mask, const void* ori_x,
                       const void* shared_x, void* y, hipStream_t stream)
{
#define MOE_DC_ARGS sh, eo, qs, ids, ei, w, erc, roff, mask, ori_x, shared_x, y, stream
    if (sh.K <= 4) return launch_elem_k<4, Q, INV>(MOE_DC_ARGS);
    return launch_elem_k<16, Q, INV>(MOE_DC_ARGS);
#undef MOE_DC_ARGS
}

// ---------------------------------------------------------------------------------------
// scatter-back: each expert-side row r < recv_offsets[W] is sent back to slot i * K + k of
// its source rank s, (s, i, k) = assist_info[r] (the sample article's combine: epOffset =
// tokenId * K + topkId).  Every rank lives in this HBM, so the slot records the row's index
// instead of a copy of its bytes; the gather then reads the row through it.
// ---------------------------------------------------------------------------------------

constexpr int kIndexThreads = 256;

__global__ __launch_bounds__(kIndexThreads) void scatter_back_index_kernel(
    const int32_t* __restrict__ assist, const int64_t* __restrict__ recv_offsets,
    int32_t* __restrict__ slot_rows, int W, int BS, int K, long long cap)
{
    const long long r = (long long)blockIdx.x * kIndexThreads + threadIdx.x;
    if (r >= cap || r >= recv_offsets[W]) return;
    const int32_t s = assist[r * 3 + 0];
    const int32_t i = assist[r * 3 + 1];
    const int32_t k = assist[r * 3 + 2];
    if (s < 0 || s >= W || i < 0 || i >= BS || k < 0 || k >= K) return;   // not a triple
    slot_rows[((long long)s * BS + i) * K + k] = (int32_t)r;
}

// ---------------------------------------------------------------------------------------
// expert-side int8 block quantization of the packed expert-output rows [0, recv_offsets[W])
// ---------------------------------------------------------------------------------------

constexpr float kInv127 = 1.0f / 127.0f;   // the reciprocal of SCALE_PARAM, one fp32 rounding

// int8 code of x / scale through fp16: each narrowing rounds to nearest even, the int8 step
// saturates at +-127, and a NaN quotient (0 / 0 in an all-zero block) gives 0.
__device__ __forceinline__ uint32_t block_code(float x, float scale)
{
    const float v = x / scale;
    const float h = (float)(_Float16)v;
    if (h != h) return 0u;
    const float r = fminf(fmaxf(__builtin_rintf(h), -127.0f), 127.0f);
    return (uint32_t)(int32_t)r & 0xFFu;
}

// The eight codes of one block, each int8(fp16(x / scale)) exactly as block_code gives it,
// with one IEEE division per block instead of one per element.  For a normal, finite scale,
// r = 1 / scale is correctly rounded and q = x * r lies within 2.5 units in the last place
// (binary32) of the correctly rounded quotient (two roundings of relative size 2^-24 each,
// against a unit of at least 2^-24 of the value), so both round to the same binary16 value
// unless a binary16 rounding midpoint lies between them.  In binary32 a midpoint between
// neighbouring binary16 values has its low 13 fraction bits equal to 0x1000; a product whose
// low 13 bits lie within 5 units of that pattern is recomputed with the exact division (near
// a power of two the neighbouring midpoints are 2^12 units away, so no other pattern can be
// crossed).  The binary16 value then rounds to an integer below 128 in magnitude: |x| <=
// amax and scale = amax * fp32(1/127) give |x / scale| <= 127 * (1 + 2^-23), so no clamp and
// no NaN arise on this path; adding 1.5 * 2^23 rounds it half to even and leaves the integer
// in the low byte.  Any other scale (zero, subnormal, infinite or NaN) takes block_code.
__device__ __forceinline__ uint2 block_codes8(const float (&f)[8], float scale)
{
    uint32_t c8[8];
    const uint32_t sb = __float_as_uint(scale);
    if (sb >= 0x00800000u && sb < 0x7F800000u) {
        const float r = 1.0f / scale;
        uint32_t near_mid = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float q = f[c] * r;
            const float h = (float)(_Float16)q;
            c8[c] = __float_as_uint(h + 12582912.0f);
            near_mid |= ((__float_as_uint(q) & 0x1FFFu) - 0xFFBu) <= 10u ? 1u << c : 0u;
        }
        if (near_mid != 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (near_mid & (1u << c)) c8[c] = block_code(f[c], scale);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) c8[c] = block_code(f[c], scale);
    }
    const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c8[3], c8[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(c8[1], c8[0], 0x0c0c0400u),
                                              0x05040100u);
    const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c8[7], c8[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(c8[5], c8[4], 0x0c0c0400u),
                                              0x05040100u);
    return make_uint2(lo, hi);
}

// One wave task = one row x 2 slots of 64 lanes; each lane owns one 8-element block.
constexpr int kQuantSlots = 2;

__global__ __launch_bounds__(kWave * kWavesPerBlock) void combine_quantize_kernel(
    const uint16_t* __restrict__ expert_out, const int64_t* __restrict__ recv_offsets,
    int8_t* __restrict__ codes, float* __restrict__ qscales, int W, int H, long long cap,
    int tasks_per_row, int tok_f16)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long long task = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const long long row = task / tasks_per_row;
    const long long rows = recv_offsets[W];
    if (row >= cap || row >= rows) return;                 // whole wave
    const int slot0 = (int)(task - row * tasks_per_row) * kQuantSlots;
    const int NV = H >> 3;
    const uint4* src = reinterpret_cast<const uint4*>(expert_out) + row * NV;
    uint4 raw[kQuantSlots];
#pragma unroll
    for (int n = 0; n < kQuantSlots; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v < NV) raw[n] = load_stream(src + v);
    }
#pragma unroll
    for (int n = 0; n < kQuantSlots; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v >= NV) continue;
        float f[8];
        if (tok_f16) {
            f[0] = f16_lo(raw[n].x); f[1] = f16_hi(raw[n].x); f[2] = f16_lo(raw[n].y);
            f[3] = f16_hi(raw[n].y); f[4] = f16_lo(raw[n].z); f[5] = f16_hi(raw[n].z);
            f[6] = f16_lo(raw[n].w); f[7] = f16_hi(raw[n].w);
        } else {
            f[0] = bf16_lo(raw[n].x); f[1] = bf16_hi(raw[n].x); f[2] = bf16_lo(raw[n].y);
            f[3] = bf16_hi(raw[n].y); f[4] = bf16_lo(raw[n].z); f[5] = bf16_hi(raw[n].z);
            f[6] = bf16_lo(raw[n].w); f[7] = bf16_hi(raw[n].w);
        }
        uint32_t amax = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t b = __float_as_uint(f[c]) & 0x7FFFFFFFu;
            amax = amax > b ? amax : b;
        }
        const float scale = __uint_as_float(amax) * kInv127;
        const uint2 packed = block_codes8(f, scale);
        store_stream(reinterpret_cast<uint2*>(codes) + row * NV + v, packed);
        __builtin_nontemporal_store(scale, qscales + row * NV + v);
    }
}

// Element-wise quantization: one workgroup per row, one element per lane; a block is 8
// adjacent lanes (the last block of a row may be short).
__global__ __launch_bounds__(kElemThreads) void combine_quantize_elem_kernel(
    const uint16_t* __restrict__ expert_out, const int64_t* __restrict__ recv_offsets,
    int8_t* __restrict__ codes, float* __restrict__ qscales, int W, int H, int tok_f16)
{
    const long long row = blockIdx.x;
    if (row >= recv_offsets[W]) return;                    // whole workgroup
    const int t = threadIdx.x;
    const int nb = (H + 7) / 8;
#pragma unroll 1
    for (int n = 0; n < kElemPerLane; ++n) {
        const int h = t + n * blockDim.x;
        if (n * (int)blockDim.x >= H) break;               // uniform across the workgroup
        const float f = h < H ? tok_lo_rt(expert_out[row * H + h], tok_f16 != 0) : 0.0f;
        const uint32_t amax = group_max_u32<8>(__float_as_uint(f) & 0x7FFFFFFFu);
        const float scale = __uint_as_float(amax) * kInv127;
        if (h >= H) continue;
        codes[row * H + h] = (int8_t)block_code(f, scale);
        if ((h & 7) == 0) qscales[row * nb + h / 8] = scale;
    }
}

}  // namespace

hipError_t launch_combine(const Shape& sh, const void* expert_out, const int32_t* expert_ids,
                          const int32_t* expand_idx, const float* expert_scales,
                          const int32_t* ep_recv_count, const int64_t* recv_offsets,
                          const uint8_t* mask, const void* ori_x, void* y, bool vectorized,
                          hipStream_t stream)
{
    if (vectorized)
        return launch_wave<0, false, false>(sh, expert_out, nullptr, expert_ids, expand_idx,
                                            expert_scales, ep_recv_count, recv_offsets, mask,
                                            ori_x, nullptr, y, stream);
    return launch_elem<0, false>(sh, expert_out, nullptr, expert_ids, expand_idx,
                                 expert_scales, ep_recv_count, recv_offsets, mask, ori_x,
                                 nullptr, y, stream);
}

hipError_t launch_combine_int8(const Shape& sh, const int8_t* codes, const float* qscales,
                               const int32_t* expert_ids, const int32_t* expand_idx,
                               const float* expert_scales, const int32_t* ep_recv_count,
                               const int64_t* recv_offsets, const uint8_t* mask,
                               const void* ori_x, void* y, bool vectorized, hipStream_t stream)
{
    // 16-element lanes need 16-byte aligned code rows and 8-byte aligned scale pairs
    const bool wide = vectorized && sh.H % 16 == 0 && sh.K <= 8 &&
                      (reinterpret_cast<uintptr_t>(codes) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(qscales) & 7u) == 0;
    if (wide) {
#define MOE_DC_ARGS sh, codes, qscales, expert_ids, expand_idx, expert_scales, ep_recv_count, \
                    recv_offsets, mask, ori_x, y, stream
        if (sh.K <= 2) return launch_int8_wide_k<2>(MOE_DC_ARGS);
        if (sh.K <= 4) return launch_int8_wide_k<4>(MOE_DC_ARGS);
        return launch_int8_wide_k<8>(MOE_DC_ARGS);
#undef MOE_DC_ARGS
    }
    if (vectorized)
        return launch_wave<1, false, false>(sh, codes, qscales, expert_ids, expand_idx,
                                            expert_scales, ep_recv_count, recv_offsets, mask,
                                            ori_x, nullptr, y, stream);
    return launch_elem<1, false>(sh, codes, qscales, expert_ids, expand_idx, expert_scales,
                                 ep_recv_count, recv_offsets, mask, ori_x, nullptr, y, stream);
}

hipError_t launch_combine_scatter(const Shape& sh, const void* expert_out,
                                  const int32_t* assist_info, const int64_t* recv_offsets,
                                  const int32_t* expert_ids, const float* expert_scales,
                                  const uint8_t* mask, const void* ori_x, const void* shared_x,
                                  void* y, int32_t* slot_rows, bool vectorized,
                                  hipStream_t stream)
{
    const unsigned blocks = (unsigned)((sh.cap + kIndexThreads - 1) / kIndexThreads);
    hipLaunchKernelGGL(scatter_back_index_kernel, dim3(blocks), dim3(kIndexThreads), 0, stream,
                       assist_info, recv_offsets, slot_rows, sh.W, sh.BS, sh.K,
                       (long long)sh.cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define MOE_DC_ARGS sh, expert_out, nullptr, expert_ids, slot_rows, expert_scales, nullptr, \
                    recv_offsets, mask, ori_x, shared_x, y, stream
    if (!vectorized) return launch_elem<0, true>(MOE_DC_ARGS);
    if (shared_x) return launch_wave<0, true, true>(MOE_DC_ARGS);
    return launch_wave<0, true, false>(MOE_DC_ARGS);
#undef MOE_DC_ARGS
}

hipError_t launch_combine_quantize(const Shape& sh, const void* expert_out,
                                   const int64_t* recv_offsets, int8_t* codes, float* qscales,
                                   bool vectorized, hipStream_t stream)
{
    if (vectorized) {
        const int slots = ((sh.H >> 3) + kWave - 1) / kWave;
        const int tasks_per_row = (slots + kQuantSlots - 1) / kQuantSlots;
        const long long tasks = (long long)sh.cap * tasks_per_row;
        const unsigned blocks = (unsigned)((tasks + kWavesPerBlock - 1) / kWavesPerBlock);
        hipLaunchKernelGGL(combine_quantize_kernel, dim3(blocks), dim3(kWave * kWavesPerBlock),
                           0, stream, static_cast<const uint16_t*>(expert_out), recv_offsets,
                           codes, qscales, sh.W, sh.H, (long long)sh.cap, tasks_per_row,
                           sh.tok_f16);
    } else {
        const int want = (sh.H + kWave - 1) / kWave * kWave;
        const int threads = want < kElemThreads ? want : kElemThreads;
        hipLaunchKernelGGL(combine_quantize_elem_kernel, dim3((unsigned)sh.cap),
                           dim3(threads), 0, stream, static_cast<const uint16_t*>(expert_out),
                           recv_offsets, codes, qscales, sh.W, sh.H, sh.tok_f16);
    }
    return hipGetLastError();
}

}  // namespace moe_dc
