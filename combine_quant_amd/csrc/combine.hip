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
// 16-byte vectors (64 for K > 8), each handled by one independent wavefront, which resolves
// the token's sources in lanes 0..K-1 and broadcasts them as wave-uniform values; expert rows
// are read and y is written with the non-temporal policy; no workgroup barrier.  Element-wise
// fallback (any H, any alignment): one workgroup per token, one element per lane.
#include "dc_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

constexpr int kNone = -1;   // inactive pick, zero expert, or unresolvable
constexpr int kCopy = -2;   // copy expert: read ori_x

// Source of pick k of token tok: its expert_out row (>= 0), kCopy for a copy expert, or
// kNone.  The row follows the design doc's addressing (§3.4.2: the owner rank's window + the
// expert's offset inside it + expand_idx), written with the dispatch outputs:
// recv_offsets[r] + the running total of ep_recv_count just before (local expert j,
// source s) + expand_idx.  Rows outside [0, cap) are treated as unresolvable.
__device__ __forceinline__ int pick_source(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ expand_idx,
    const int32_t* __restrict__ ep_recv_count, const int64_t* __restrict__ recv_offsets,
    const uint8_t* __restrict__ mask, int mask_kind, int W, int E, int L, int K, int zero_end,
    int id_end, long long cap, long long tok, int s, int k)
{
    const long long p = tok * K + k;
    const int32_t e = ids[p];
    const bool on = mask_kind == 0 || (mask_kind == 1 ? mask[tok] != 0 : mask[p] != 0);
    if (!on || e < 0) return kNone;
    if (e < E) {
        const int32_t ord = expand_idx[p];
        if (ord < 0) return kNone;
        const int r = e / L;
        const int j = e - r * L;
        const long long flat = (long long)j * W + s;
        const long long base =
            flat == 0 ? 0 : (long long)ep_recv_count[(long long)r * L * W + flat - 1];
        const long long row = (long long)recv_offsets[r] + base + ord;
        return (row >= 0 && row < cap) ? (int)row : kNone;
    }
    return (e >= zero_end && e < id_end) ? kCopy : kNone;
}

// acc[c] = acc[c] + w * element c of eight bf16 values (one multiply, one add each)
__device__ __forceinline__ void accumulate8(uint4 v, float w, float (&acc)[8])
{
    const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = acc[c] + w * f[c];
}

constexpr int kWavesPerBlock = 4;

// 64-vector slots of one token per wave task: two (16 row loads in flight per lane at K=8);
// one for K > 8, where two would need 32 loads' worth of registers and halve occupancy.
constexpr int slots_per_task(int kmax) { return kmax > 8 ? 1 : 2; }

// One wave task = one token x SLOTS slots of 64 16-byte vectors.  A token's row is
// split across several independent waves (each resolves the token's K sources itself), so a
// launch is many short tasks: the hardware keeps every SIMD busy to the end instead of
// leaving a long, thinly occupied last round of whole-token waves.
template <int KMAX, int SLOTS>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void combine_wave_kernel(
    const uint16_t* __restrict__ expert_out, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const float* __restrict__ weights,
    const int32_t* __restrict__ ep_recv_count, const int64_t* __restrict__ recv_offsets,
    const uint8_t* __restrict__ mask, int mask_kind, const uint16_t* __restrict__ ori_x,
    uint16_t* __restrict__ y, int W, int E, int L, int BS, int H, int K, int zero_end,
    int id_end, long long cap, long long T, int tasks_per_token)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long long task = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const long long tok = task / tasks_per_token;
    if (tok >= T) return;                                  // whole wave
    const int slot0 = (int)(task - tok * tasks_per_token) * SLOTS;
    const int s = (int)(tok / BS);
    const int NV = H >> 3;

    int src = kNone;
    float wk = 0.0f;
    if (lane < K) {
        src = pick_source(ids, expand_idx, ep_recv_count, recv_offsets, mask, mask_kind, W, E,
                          L, K, zero_end, id_end, cap, tok, s, lane);
        wk = weights[tok * K + lane];
    }
    int srcs[KMAX];
    float ws[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        srcs[k] = k < K ? lane_value(src, k) : kNone;
        ws[k] = lane_value(wk, k);
    }

    const uint4* eo = reinterpret_cast<const uint4*>(expert_out);
    const uint4* self = ori_x ? reinterpret_cast<const uint4*>(ori_x) + tok * NV : nullptr;
    uint4* yr = reinterpret_cast<uint4*>(y) + tok * NV;
    uint4 buf[SLOTS][KMAX];
#pragma unroll
    for (int n = 0; n < SLOTS; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v < NV) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (srcs[k] >= 0) buf[n][k] = load_stream(eo + (long long)srcs[k] * NV + v);
                else if (srcs[k] == kCopy) buf[n][k] = self[v];
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
            for (int k = 0; k < KMAX; ++k)
                if (srcs[k] != kNone) accumulate8(buf[n][k], ws[k], acc);
            store_stream(yr + v,
                         make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                    pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])));
        }
    }
}

template <int KMAX>
hipError_t launch_wave_k(const Shape& sh, const void* expert_out, const int32_t* ids,
                         const int32_t* expand_idx, const float* w, const int32_t* erc,
                         const int64_t* roff, const uint8_t* mask, const void* ori_x, void* y,
                         hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    const int slots = ((sh.H >> 3) + kWave - 1) / kWave;
    constexpr int kSlots = slots_per_task(KMAX);
    const int tasks_per_token = (slots + kSlots - 1) / kSlots;
    const long long tasks = T * tasks_per_token;
    const unsigned blocks = (unsigned)((tasks + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL((combine_wave_kernel<KMAX, kSlots>), dim3(blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream,
                       static_cast<const uint16_t*>(expert_out), ids, expand_idx, w, erc, roff,
                       mask, sh.mask_kind, static_cast<const uint16_t*>(ori_x),
                       static_cast<uint16_t*>(y), sh.W, sh.E, sh.L, sh.BS, sh.H, sh.K,
                       sh.zero_end, sh.id_end, (long long)sh.cap, T, tasks_per_token);
    return hipGetLastError();
}

hipError_t launch_wave(const Shape& sh, const void* eo, const int32_t* ids, const int32_t* ei,
                       const float* w, const int32_t* erc, const int64_t* roff,
                       const uint8_t* mask, const void* ori_x, void* y, hipStream_t stream)
{
    if (sh.K <= 2) return launch_wave_k<2>(sh, eo, ids, ei, w, erc, roff, mask, ori_x, y, stream);
    if (sh.K <= 4) return launch_wave_k<4>(sh, eo, ids, ei, w, erc, roff, mask, ori_x, y, stream);
    if (sh.K <= 8) return launch_wave_k<8>(sh, eo, ids, ei, w, erc, roff, mask, ori_x, y, stream);
    return launch_wave_k<16>(sh, eo, ids, ei, w, erc, roff, mask, ori_x, y, stream);
}

constexpr int kElemThreads = 1024;
constexpr int kElemPerLane = 8;      // H <= 8192 = 1024 lanes x 8

template <int KMAX>
__global__ __launch_bounds__(kElemThreads) void combine_elem_kernel(
    const uint16_t* __restrict__ expert_out, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const float* __restrict__ weights,
    const int32_t* __restrict__ ep_recv_count, const int64_t* __restrict__ recv_offsets,
    const uint8_t* __restrict__ mask, int mask_kind, const uint16_t* __restrict__ ori_x,
    uint16_t* __restrict__ y, int W, int E, int L, int BS, int H, int K, int zero_end,
    int id_end, long long cap)
{
    __shared__ int src_of[KMAX];
    __shared__ float w_of[KMAX];
    const long long tok = blockIdx.x;
    const int s = (int)(tok / BS);
    const int t = threadIdx.x;
    if (t < K) {
        src_of[t] = pick_source(ids, expand_idx, ep_recv_count, recv_offsets, mask, mask_kind,
                                W, E, L, K, zero_end, id_end, cap, tok, s, t);
        w_of[t] = weights[tok * K + t];
    }
    __syncthreads();
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
            const uint16_t b = src >= 0 ? expert_out[(long long)src * H + h] : self[h];
            acc = acc + w_of[k] * bf16_lo(b);
        }
        yr[h] = (uint16_t)f32_to_bf16_rne(acc);
    }
}

template <int KMAX>
hipError_t launch_elem_k(const Shape& sh, const void* expert_out, const int32_t* ids,
                         const int32_t* expand_idx, const float* w, const int32_t* erc,
                         const int64_t* roff, const uint8_t* mask, const void* ori_x, void* y,
                         hipStream_t stream)
{
    const int want = (sh.H + kWave - 1) / kWave * kWave;
    const int threads = want < kElemThreads ? want : kElemThreads;
    const long long T = (long long)sh.W * sh.BS;
    hipLaunchKernelGGL((combine_elem_kernel<KMAX>), dim3((unsigned)T), dim3(threads), 0,
                       stream, static_cast<const uint16_t*>(expert_out), ids, expand_idx, w,
                       erc, roff, mask, sh.mask_kind, static_cast<const uint16_t*>(ori_x),
                       static_cast<uint16_t*>(y), sh.W, sh.E, sh.L, sh.BS, sh.H, sh.K,
                       sh.zero_end, sh.id_end, (long long)sh.cap);
    return hipGetLastError();
}

hipError_t launch_elem(const Shape& sh, const void* eo, const int32_t* ids, const int32_t* ei,
                       const float* w, const int32_t* erc, const int64_t* roff,
                       const uint8_t* mask, const void* ori_x, void* y, hipStream_t stream)
{
    if (sh.K <= 4) return launch_elem_k<4>(sh, eo, ids, ei, w, erc, roff, mask, ori_x, y, stream);
    return launch_elem_k<16>(sh, eo, ids, ei, w, erc, roff, mask, ori_x, y, stream);
}

}  // namespace

hipError_t launch_combine(const Shape& sh, const void* expert_out, const int32_t* expert_ids,
                          const int32_t* expand_idx, const float* expert_scales,
                          const int32_t* ep_recv_count, const int64_t* recv_offsets,
                          const uint8_t* mask, const void* ori_x, void* y, bool vectorized,
                          hipStream_t stream)
{
    if (vectorized)
        return launch_wave(sh, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
                           recv_offsets, mask, ori_x, y, stream);
    return launch_elem(sh, expert_out, expert_ids, expand_idx, expert_scales, ep_recv_count,
                       recv_offsets, mask, ori_x, y, stream);
}

}  // namespace moe_dc
