// route_device.h -- device helpers of the routing steps (route, scan and the small-batch
// routing inside the scatter launch): which picks are routed, which break the id contract,
// and a workgroup-wide inclusive scan.
#pragma once

#include "dc_device.h"

namespace moe_dc {

// Inclusive scan of one int per thread across the workgroup (wave shuffles + LDS).
// `wave_tot` holds one word per wave; the call contains one barrier.
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* wave_tot)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int32_t o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wave_tot[wave] = v;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    return v + before;
}

// Expert of pick k of token tok when the pick is routed -- active under the mask (kind 1:
// mask[tok], kind 2: mask[tok*K + k], nonzero = active) and 0 <= id < E -- else -1.
__device__ __forceinline__ int32_t routed_expert(const int32_t* __restrict__ ids,
                                                 const uint8_t* __restrict__ mask,
                                                 int mask_kind, int K, int E, long long tok,
                                                 int k)
{
    const long long p = tok * K + k;
    const int32_t v = ids[p];
    const bool on = (mask_kind != 1 || mask[tok] != 0) && (mask_kind != 2 || mask[p] != 0);
    return on && (uint32_t)v < (uint32_t)E ? v : -1;
}

// 1 when pick k of token tok is active under the mask but its id lies outside [0, id_end)
// (a contract violation the id check counts), else 0.
__device__ __forceinline__ int32_t bad_pick(const int32_t* __restrict__ ids,
                                            const uint8_t* __restrict__ mask, int mask_kind,
                                            int K, int id_end, long long tok, int k)
{
    const long long p = tok * K + k;
    const int32_t v = ids[p];
    const bool on = (mask_kind != 1 || mask[tok] != 0) && (mask_kind != 2 || mask[p] != 0);
    return on && (v < 0 || v >= id_end) ? 1 : 0;
}

}  // namespace moe_dc
