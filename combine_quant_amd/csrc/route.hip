// route.hip -- routing ordinals and receive-side prefix sums on gfx950.
//
// expand_idx of a pick (s, i, k) with expert e is the number of picks of source rank s that
// come before it in row-major (token, pick) order and chose e (MoeDistributeDispatch design
// doc, §2.2.2, index computation).  The pages compute it with a serial running count; here
// it is computed in parallel and deterministically, without relying on the order in which
// atomics land:
//
//   * one workgroup per (source rank s, group of 32 experts), one lane per token, builds in
//     LDS a bitmap hit[e][i/32] with bit i%32 set when token i picked e at least once, plus
//     extra[e][i/32] = picks beyond the first made by the tokens of that 32-token word
//     (duplicates inside a token; the pages' own example draws ids with replacement).  OR
//     and ADD commute, so the LDS contents do not depend on thread timing.
//   * an exclusive running popcount over each expert's words turns this into
//       ordinal(i, k) = #hits in earlier words + extras in earlier words
//                     + #hits of earlier tokens in the same word (masked popcount)
//                     + duplicates of e earlier in token i
//                     + extras of earlier tokens in the same word (only if that word has any)
//   * the per-(expert, source) totals go to the workspace at e*W + s;
//   * a token whose picks are all different (the usual case) needs none of the duplicate
//     bookkeeping; a token with a repeated expert takes the exact slower branch.
//
// The receive-side scan (design doc §2.4: transpose the W x L receive matrix, then a
// row-major running sum) is one workgroup.  Because the workspace keeps the counts in the
// flat order e*W + s, which is the (local expert j, source s) order of every receiver's
// ep_recv_count laid end to end, one exclusive scan of that flat array yields every segment
// base and, by differences, every output.
#include "dc_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

constexpr int kRouteExperts = 32;     // experts per routing workgroup
constexpr int kScanThreads = 1024;    // >= E (E <= 1024 is validated)
constexpr int kScanLdsCounts = 16384; // counts staged in LDS by the scan (64 KiB)

// Expert id of each pick of token `tok`, or -1 when the pick is not routed (inactive,
// special expert, or an id outside [0, E)).
template <int KMAX>
__device__ __forceinline__ void routed_picks(const int32_t* __restrict__ ids,
                                             const uint8_t* __restrict__ mask, int mask_kind,
                                             int K, int E, long long tok, int32_t (&e)[KMAX])
{
    const bool tok_on = mask_kind != 1 || mask[tok] != 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int32_t v = -1;
        if (k < K) {
            v = ids[tok * K + k];
            const bool on = tok_on && (mask_kind != 2 || mask[tok * K + k] != 0);
            if (!on || v < 0 || v >= E) v = -1;
        }
        e[k] = v;
    }
}

template <int KMAX>
__global__ __launch_bounds__(512) void route_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask, int mask_kind, int W,
    int E, int BS, int K, int nwords, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ seg)
{
    extern __shared__ uint32_t lds[];
    const int s = blockIdx.x;
    const int e_lo = blockIdx.y * kRouteExperts;
    const int ne = min(kRouteExperts, E - e_lo);
    const int n = ne * nwords;
    uint32_t* hit = lds;               // [ne][nwords]
    uint32_t* extra = hit + n;         // [ne][nwords]
    uint32_t* hit_pre = extra + n;     // [ne][nwords] exclusive running popcount of hit
    uint32_t* extra_pre = hit_pre + n; // [ne][nwords] exclusive running sum of extra

    // one lane per token; its picks stay in registers for both passes
    const int i = threadIdx.x;
    const long long tok = (long long)s * BS + i;
    int32_t e[KMAX];
    bool distinct = true;
    if (i < BS) {
        routed_picks<KMAX>(ids, mask, mask_kind, K, E, tok, e);
#pragma unroll
        for (int a = 0; a < KMAX; ++a)
#pragma unroll
            for (int b = a + 1; b < KMAX; ++b)
                if (e[a] >= 0 && e[a] == e[b]) distinct = false;
    }
    for (int w = threadIdx.x; w < 2 * n; w += blockDim.x) lds[w] = 0;
    __syncthreads();

    const int wd = i >> 5;
    const uint32_t bit = 1u << (i & 31);
    if (i < BS) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int32_t ek = e[k];
            if (ek < e_lo || ek >= e_lo + ne) continue;
            const int word = (ek - e_lo) * nwords + wd;
            if (distinct) {
                atomicOr(&hit[word], bit);
                continue;
            }
            bool first = true;
            uint32_t mult = 1;
#pragma unroll
            for (int k2 = 0; k2 < KMAX; ++k2) {
                if (k2 != k && e[k2] == ek) {
                    ++mult;
                    if (k2 < k) first = false;
                }
            }
            if (first) {
                atomicOr(&hit[word], bit);
                if (mult > 1) atomicAdd(&extra[word], mult - 1);
            }
        }
    }
    __syncthreads();

    // exclusive running totals over each expert's words: one thread per (expert, word),
    // summing the words before it (at most 15) with independent LDS reads
    for (int q = threadIdx.x; q < n; q += blockDim.x) {
        const int el = q / nwords;
        const int w = q - el * nwords;
        uint32_t rp = 0, rx = 0;
        for (int w2 = 0; w2 < w; ++w2) {
            rp += __popc(hit[el * nwords + w2]);
            rx += extra[el * nwords + w2];
        }
        hit_pre[q] = rp;
        extra_pre[q] = rx;
        if (w == nwords - 1)
            seg[(long long)(e_lo + el) * W + s] = (int32_t)(rp + __popc(hit[q]) + rx + extra[q]);
    }
    __syncthreads();

    if (i >= BS) return;
    const uint32_t below = bit - 1u;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int32_t ek = e[k];
        if (k >= K) continue;
        if (ek < 0) {
            if (blockIdx.y == 0) expand_idx[tok * K + k] = -1;
            continue;
        }
        if (ek < e_lo || ek >= e_lo + ne) continue;
        const int word = (ek - e_lo) * nwords + wd;
        uint32_t ord = hit_pre[word] + extra_pre[word] + __popc(hit[word] & below);
        if (!distinct) {
#pragma unroll
            for (int k2 = 0; k2 < KMAX; ++k2)
                if (k2 < k && e[k2] == ek) ++ord;
        }
        if (extra[word] != 0) {
            // earlier tokens of this 32-token word that picked ek more than once
            uint32_t bits = hit[word] & below;
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1u;
                int32_t e2[KMAX];
                routed_picks<KMAX>(ids, mask, mask_kind, K, E, (long long)s * BS + wd * 32 + b,
                                   e2);
                uint32_t c = 0;
#pragma unroll
                for (int k2 = 0; k2 < KMAX; ++k2)
                    if (e2[k2] == ek) ++c;
                ord += c - 1u;
            }
        }
        expand_idx[tok * K + k] = (int32_t)ord;
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

// Receive-side scan when the W*E counts fit in LDS.  In the flat order f = e*W + s (expert
// major, source minor) the exclusive running total ex[f] is exactly the first packed row of
// segment (e, s), and every output is a difference of two entries of ex:
//   ep_recv_count[f]       = ex[f+1] - ex[first f of e's rank]
//   recv_offsets[r]        = ex[r*L*W],   recv_offsets[W] = ex[W*E]
//   expert_token_nums[e]   = ex[(e+1)*W] - ex[e*W]            (counts, type 1)
//                          = ex[(e+1)*W] - ex[r*L*W]          (running sum, type 0)
// One block-wide scan (each thread a run of consecutive entries, wave shuffles, LDS across
// waves), then coalesced stores.
__global__ __launch_bounds__(kScanThreads) void scan_flat_kernel(
    int W, int E, int L, int etn_type, int32_t* __restrict__ seg,
    int32_t* __restrict__ ep_recv_count, int64_t* __restrict__ expert_token_nums,
    int64_t* __restrict__ recv_offsets)
{
    extern __shared__ int32_t ex[];          // N + 1 entries
    __shared__ int32_t wave_tot[kScanThreads / kWave];
    const int N = E * W;
    const int t = threadIdx.x;
    for (int f = t; f < N; f += blockDim.x) ex[f] = seg[f];
    __syncthreads();
    const int per = (N + blockDim.x - 1) / blockDim.x;
    const int lo = min(N, t * per);
    const int hi = min(N, lo + per);
    int32_t run = 0;
    for (int f = lo; f < hi; ++f) run += ex[f];
    const int32_t incl = block_inclusive_scan(run, wave_tot);
    int32_t acc = incl - run;
    for (int f = lo; f < hi; ++f) {
        const int32_t c = ex[f];
        ex[f] = acc;
        acc += c;
    }
    if (t == blockDim.x - 1) ex[N] = incl;
    __syncthreads();
    for (int f = t; f < N; f += blockDim.x) {
        const int e = f / W;
        const int rank_first = (e / L) * L * W;
        seg[f] = ex[f];
        ep_recv_count[f] = ex[f + 1] - ex[rank_first];
    }
    for (int e = t; e < E; e += blockDim.x) {
        const int rank_first = (e / L) * L * W;
        expert_token_nums[e] =
            (int64_t)(ex[(e + 1) * W] - (etn_type == 0 ? ex[rank_first] : ex[e * W]));
    }
    for (int r = t; r <= W; r += blockDim.x) recv_offsets[r] = ex[r * L * W];
}

// Receive-side scan for shapes whose counts exceed the LDS budget: one thread per expert
// walks its W sources in global memory (each thread reads and rewrites only its own
// entries).
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
        for (int s = 0; s < W; ++s) total += seg[(long long)e * W + s];
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
        const long long f = (long long)e * W + s;   // = r*L*W + j*W + s
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
    const int threads = (sh.BS + kWave - 1) / kWave * kWave;      // one lane per token
    const dim3 grid(sh.W, groups);
#define MOE_DC_ROUTE(KM)                                                                        \
    hipLaunchKernelGGL(route_kernel<KM>, grid, dim3(threads), lds, stream, expert_ids, mask,  \
                       sh.mask_kind, sh.W, sh.E, sh.BS, sh.K, nwords, expand_idx, seg)
    if (sh.K <= 2) MOE_DC_ROUTE(2);
    else if (sh.K <= 4) MOE_DC_ROUTE(4);
    else if (sh.K <= 8) MOE_DC_ROUTE(8);
    else MOE_DC_ROUTE(16);
#undef MOE_DC_ROUTE
    return hipGetLastError();
}

hipError_t launch_scan(const Shape& sh, int32_t* seg, int32_t* ep_recv_count,
                       int64_t* expert_token_nums, int64_t* recv_offsets, hipStream_t stream)
{
    const long long n = (long long)sh.E * sh.W;
    if (n <= kScanLdsCounts) {
        hipLaunchKernelGGL(scan_flat_kernel, dim3(1), dim3(kScanThreads),
                           (n + 1) * sizeof(int32_t), stream, sh.W, sh.E, sh.L, sh.etn_type, seg,
                           ep_recv_count, expert_token_nums, recv_offsets);
    } else {
        const int threads = ((sh.E + kWave - 1) / kWave) * kWave;
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(threads), 0, stream, sh.W, sh.E, sh.L,
                           sh.etn_type, seg, ep_recv_count, expert_token_nums, recv_offsets);
    }
    return hipGetLastError();
}

}  // namespace moe_dc
