// route.hip -- routing ordinals and receive-side prefix sums on gfx950.
//
// expand_idx of a pick (s, i, k) with expert e is the number of picks of source rank s that
// come before it in row-major (token, pick) order and chose e (MoeDistributeDispatch design
// doc, §2.2.2, index computation).  The pages compute it with a serial running count; here
// it is computed in parallel and deterministically, without relying on the order in which
// atomics land:
//
//   * one workgroup per (source rank s, group of 64 experts) builds, in LDS, a bitmap
//     hit[e][i/32] with bit i%32 set when token i picked e at least once, plus extra[e][i/32]
//     = picks beyond the first made by the tokens of that 32-token word (duplicates inside a
//     token; the pages' own example draws ids with replacement).  OR and ADD commute, so the
//     LDS contents do not depend on thread timing.
//   * an exclusive running popcount over each expert's words turns this into
//       ordinal(i, k) = #hits in earlier words + extras in earlier words
//                     + #hits of earlier tokens in the same word (masked popcount)
//                     + duplicates of e earlier in token i
//                     + extras of earlier tokens in the same word (only if that word has any)
//   * the per-(expert, source) totals go to the workspace at e*W + s.
//
// The receive-side scan (design doc §2.4: transpose the W x L receive matrix, then a
// row-major running sum) is one workgroup over the experts: each thread owns one expert
// and walks the W sources serially, which is exactly the (j, s) flat order of ep_recv_count.
#include "dc_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteExperts = 64;     // experts per routing workgroup
constexpr int kScanThreads = 1024;    // >= E (E <= 1024 is validated)

// Expert id of each pick of token `tok`, or -1 when the pick is not routed (inactive,
// special expert, or an id outside [0, E)).
__device__ __forceinline__ void routed_picks(const int32_t* __restrict__ ids,
                                             const uint8_t* __restrict__ mask, int mask_kind,
                                             int K, int E, size_t tok, int32_t (&e)[kMaxK])
{
    const bool tok_on = mask_kind != 1 || mask[tok] != 0;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        int32_t v = -1;
        if (k < K) {
            v = ids[tok * K + k];
            bool on = tok_on && (mask_kind != 2 || mask[tok * K + k] != 0);
            if (!on || v < 0 || v >= E) v = -1;
        }
        e[k] = v;
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask, int mask_kind, int W,
    int E, int BS, int K, int nwords, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ seg)
{
    extern __shared__ uint32_t lds[];
    const int s = blockIdx.x;
    const int e_lo = blockIdx.y * kRouteExperts;
    const int ne = min(kRouteExperts, E - e_lo);
    const int n = ne * nwords;
    uint32_t* hit = lds;              // [ne][nwords]
    uint32_t* extra = hit + n;        // [ne][nwords]
    uint32_t* hit_pre = extra + n;    // [ne][nwords] exclusive running popcount of hit
    uint32_t* extra_pre = hit_pre + n;// [ne][nwords] exclusive running sum of extra

    for (int w = threadIdx.x; w < 2 * n; w += blockDim.x) lds[w] = 0;
    __syncthreads();

    for (int i = threadIdx.x; i < BS; i += blockDim.x) {
        const size_t tok = (size_t)s * BS + i;
        int32_t e[kMaxK];
        routed_picks(ids, mask, mask_kind, K, E, tok, e);
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            const int32_t ek = e[k];
            if (k >= K || ek < e_lo || ek >= e_lo + ne) continue;
            bool first = true;
            uint32_t mult = 1;
#pragma unroll
            for (int k2 = 0; k2 < kMaxK; ++k2) {
                if (k2 != k && k2 < K && e[k2] == ek) {
                    ++mult;
                    if (k2 < k) first = false;
                }
            }
            if (first) {
                const int word = (ek - e_lo) * nwords + (i >> 5);
                atomicOr(&hit[word], 1u << (i & 31));
                if (mult > 1) atomicAdd(&extra[word], mult - 1);
            }
        }
    }
    __syncthreads();

    for (int el = threadIdx.x; el < ne; el += blockDim.x) {
        uint32_t rp = 0, rx = 0;
        for (int w = 0; w < nwords; ++w) {
            const int word = el * nwords + w;
            hit_pre[word] = rp;
            extra_pre[word] = rx;
            rp += __popc(hit[word]);
            rx += extra[word];
        }
        seg[(size_t)(e_lo + el) * W + s] = (int32_t)(rp + rx);
    }
    __syncthreads();

    for (int i = threadIdx.x; i < BS; i += blockDim.x) {
        const size_t tok = (size_t)s * BS + i;
        int32_t e[kMaxK];
        routed_picks(ids, mask, mask_kind, K, E, tok, e);
        const uint32_t below = (1u << (i & 31)) - 1u;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            if (k >= K) continue;
            const int32_t ek = e[k];
            if (ek < 0) {
                if (blockIdx.y == 0) expand_idx[tok * K + k] = -1;
                continue;
            }
            if (ek < e_lo || ek >= e_lo + ne) continue;
            const int wd = i >> 5;
            const int word = (ek - e_lo) * nwords + wd;
            uint32_t ord = hit_pre[word] + extra_pre[word] + __popc(hit[word] & below);
#pragma unroll
            for (int k2 = 0; k2 < kMaxK; ++k2)
                if (k2 < k && e[k2] == ek) ++ord;
            if (extra[word] != 0) {
                // earlier tokens of this word that picked ek more than once
                uint32_t bits = hit[word] & below;
                while (bits) {
                    const int b = __ffs(bits) - 1;
                    bits &= bits - 1u;
                    int32_t e2[kMaxK];
                    routed_picks(ids, mask, mask_kind, K, E, (size_t)s * BS + wd * 32 + b, e2);
                    uint32_t c = 0;
#pragma unroll
                    for (int k2 = 0; k2 < kMaxK; ++k2)
                        if (k2 < K && e2[k2] == ek) ++c;
                    ord += c - 1u;
                }
            }
            expand_idx[tok * K + k] = (int32_t)ord;
        }
    }
}

// Inclusive scan of one int per thread across the workgroup (wave shuffles + LDS).
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

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    int W, int E, int L, int etn_type, int32_t* __restrict__ seg,
    int32_t* __restrict__ ep_recv_count, int64_t* __restrict__ expert_token_nums,
    int64_t* __restrict__ recv_offsets)
{
    __shared__ int32_t wave_tot[kScanThreads / kWave];
    __shared__ int32_t expert_excl[kScanThreads];
    const int e = threadIdx.x;
    int32_t total = 0;
    if (e < E)
        for (int s = 0; s < W; ++s) total += seg[(size_t)e * W + s];
    const int32_t incl = block_inclusive_scan(total, wave_tot);
    const int32_t excl = incl - total;
    expert_excl[e] = excl;
    __syncthreads();
    if (e >= E) return;
    const int r = e / L;
    const int j = e - r * L;
    const int32_t rank_base = expert_excl[r * L];
    if (j == 0) recv_offsets[r] = rank_base;
    if (e == E - 1) recv_offsets[W] = incl;
    expert_token_nums[e] = etn_type == 0 ? (int64_t)(incl - rank_base) : (int64_t)total;
    int32_t run = excl;
    for (int s = 0; s < W; ++s) {
        const size_t f = (size_t)e * W + s;   // = r*L*W + j*W + s
        const int32_t c = seg[f];
        seg[f] = run;
        run += c;
        ep_recv_count[f] = run - rank_base;
    }
}

}  // namespace

hipError_t launch_route(const Shape& sh, const int32_t* expert_ids, const uint8_t* mask,
                        int32_t* expand_idx, int32_t* seg, hipStream_t stream)
{
    const int nwords = (sh.BS + 31) / 32;
    const int groups = (sh.E + kRouteExperts - 1) / kRouteExperts;
    const int ne = sh.E < kRouteExperts ? sh.E : kRouteExperts;
    const size_t lds = (size_t)4 * ne * nwords * sizeof(uint32_t);
    hipLaunchKernelGGL(route_kernel, dim3(sh.W, groups), dim3(kRouteThreads), lds, stream,
                       expert_ids, mask, sh.mask_kind, sh.W, sh.E, sh.BS, sh.K, nwords,
                       expand_idx, seg);
    return hipGetLastError();
}

hipError_t launch_scan(const Shape& sh, int32_t* seg, int32_t* ep_recv_count,
                       int64_t* expert_token_nums, int64_t* recv_offsets, hipStream_t stream)
{
    const int threads = ((sh.E + kWave - 1) / kWave) * kWave;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(threads), 0, stream, sh.W, sh.E, sh.L,
                       sh.etn_type, seg, ep_recv_count, expert_token_nums, recv_offsets);
    return hipGetLastError();
}

}  // namespace moe_dc
