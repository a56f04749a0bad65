// route.hip -- routing ordinals and receive-side prefix sums on gfx950.
//
// expand_idx of a pick (s, i, k) with expert e is the number of picks of source rank s that
// come before it in row-major (token, pick) order and chose e (MoeDistributeDispatch design
// doc, §2.2.2, index computation).  The pages compute it with a serial running count; here
// it is computed in parallel and deterministically, without relying on the order in which
// atomics land:
//
//   * one workgroup per (source rank s, group of experts; about one workgroup per CU), one
//     lane per token, builds in LDS a bitmap hit[e][i/32] with bit i%32 set when token i
//     picked e at least once, plus extra[e][i/32] = picks beyond the first made by the tokens
//     of that 32-token word (duplicates inside a token; the pages' own example draws ids
//     with replacement).  OR and ADD commute, so the LDS contents do not depend on thread
//     timing; and because bit i belongs to token i alone, the old value returned by the OR
//     tells the lane whether its token already picked that expert.
//   * an exclusive running popcount over each expert's words turns this into
//       ordinal(i, k) = #hits in earlier words + extras in earlier words
//                     + #hits of earlier tokens in the same word (masked popcount)
//                     + (only in words with extras) this token's earlier picks of e and the
//                       repeats of the earlier tokens of the word
//   * the per-(expert, source) totals go to the workspace at e*W + s.
//
// The receive-side scan (design doc §2.4: transpose the W x L receive matrix, then a
// row-major running sum) is one workgroup.  Because the workspace keeps the counts in the
// flat order e*W + s, which is the (local expert j, source s) order of every receiver's
// ep_recv_count laid end to end, one exclusive scan of that flat array yields every segment
// base and, by differences, every output.
#include "dc_device.h"
#include "route_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

constexpr int kMaxRouteExperts = 256; // experts per routing workgroup, at most
constexpr int kScanThreads = 1024;    // >= E (E <= 1024 is validated)
constexpr int kScanLdsCounts = 16384; // counts staged in LDS by the scan (64 KiB)
constexpr int kGroupCounts = 15872;   // entries per group of ranks in the two-launch scan: with
                                      // its padding, under 64 KiB of LDS

// Expert id of each pick of token `tok`, or -1 when the pick is not routed (inactive,
// special expert, or an id outside [0, E)).  Every load of the token (ids, mask bytes) is
// issued before any of them is used, so they are in flight together.
template <int KMAX>
__device__ __forceinline__ void routed_picks(const int32_t* __restrict__ ids,
                                             const uint8_t* __restrict__ mask, int mask_kind,
                                             int K, int E, long long tok, int32_t (&e)[KMAX])
{
    int32_t v[KMAX];
    uint8_t m[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) v[k] = k < K ? ids[tok * K + k] : -1;
    if (mask_kind == 2) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) m[k] = k < K ? mask[tok * K + k] : 0;
    }
    const bool tok_on = mask_kind != 1 || mask[tok] != 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const bool on = tok_on && (mask_kind != 2 || m[k] != 0);
        e[k] = (k < K && on && (uint32_t)v[k] < (uint32_t)E) ? v[k] : -1;
    }
}

// Same, for K == KMAX with KMAX a multiple of 4 and 16-byte aligned ids: 16-byte loads.
// An id is routed when its pick is active and 0 <= id < E (one unsigned compare).
template <int KMAX>
__device__ __forceinline__ void routed_picks_vec(const int32_t* __restrict__ ids,
                                                 const uint8_t* __restrict__ mask, int mask_kind,
                                                 int E, long long tok, int32_t (&e)[KMAX])
{
    const int4* p = reinterpret_cast<const int4*>(ids + tok * KMAX);
    int4 v[KMAX >= 4 ? KMAX / 4 : 1];
    uint8_t m[KMAX];
#pragma unroll
    for (int q = 0; q < KMAX / 4; ++q) v[q] = p[q];
    if (mask_kind == 2) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) m[k] = mask[tok * KMAX + k];
    }
    const bool tok_on = mask_kind != 1 || mask[tok] != 0;
#pragma unroll
    for (int q = 0; q < KMAX / 4; ++q) {
        const int32_t r[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int k = 4 * q + c;
            const bool on = tok_on && (mask_kind != 2 || m[k] != 0);
            e[k] = (on && (uint32_t)r[c] < (uint32_t)E) ? r[c] : -1;
        }
    }
}

// bad_counts (null unless ids are checked): the workgroups of expert group 0 store their
// source rank's number of active picks whose id lies outside [0, id_end).
template <int KMAX, bool VEC_IDS>
__global__ __launch_bounds__(512) void route_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask, int mask_kind, int W,
    int E, int BS, int K, int nwords, int group, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ seg, int32_t* __restrict__ bad_counts, int id_end)
{
    extern __shared__ uint32_t lds[];
    __shared__ int32_t bad_lds;
    const int s = blockIdx.x;
    const int e_lo = blockIdx.y * group;
    const int ne = min(group, E - e_lo);
    const int n = ne * nwords;
    uint32_t* hit = lds;               // [ne][nwords]
    uint32_t* extra = hit + n;         // [ne][nwords]
    uint32_t* hit_pre = extra + n;     // [ne][nwords] exclusive running popcount of hit
    uint32_t* extra_pre = hit_pre + n; // [ne][nwords] exclusive running sum of extra

    // one lane per token; its picks stay in registers for both passes
    const int i = threadIdx.x;
    const long long tok = (long long)s * BS + i;
    int32_t e[KMAX];
    if (i < BS) {
        if (VEC_IDS) routed_picks_vec<KMAX>(ids, mask, mask_kind, E, tok, e);
        else routed_picks<KMAX>(ids, mask, mask_kind, K, E, tok, e);
    }
    for (int w = threadIdx.x; w < 2 * n; w += blockDim.x) lds[w] = 0;
    const bool check = bad_counts != nullptr && blockIdx.y == 0;     // uniform
    if (threadIdx.x == 0) bad_lds = 0;
    __syncthreads();
    if (check && i < BS) {
        int32_t c = 0;
        for (int k = 0; k < K; ++k) c += bad_pick(ids, mask, mask_kind, K, id_end, tok, k);
        if (c != 0) atomicAdd(&bad_lds, c);
    }

    // Bit i of a word belongs to token i alone and this lane walks its picks in k order, so
    // the value atomicOr returns says whether this token already picked the expert: each
    // repeat counts one extra pick for the word.
    const int wd = i >> 5;
    const uint32_t bit = 1u << (i & 31);
    if (i < BS) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int32_t ek = e[k];
            if (ek < e_lo || ek >= e_lo + ne) continue;
            const int word = (ek - e_lo) * nwords + wd;
            if (atomicOr(&hit[word], bit) & bit) atomicAdd(&extra[word], 1u);
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
    if (check && threadIdx.x == 0) bad_counts[s] = bad_lds;

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
        if (extra[word] != 0) {
            // some token of this 32-token word picked ek more than once: add this token's
            // own earlier picks of ek, and the repeats of the earlier tokens of the word
#pragma unroll
            for (int k2 = 0; k2 < KMAX; ++k2)
                if (k2 < k && e[k2] == ek) ++ord;
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

// Receive-side scan when the W*E counts fit in LDS.  In the flat order f = e*W + s (expert
// major, source minor) the exclusive running total ex[f] is exactly the first packed row of
// segment (e, s), and every output is a difference of two entries of ex:
//   ep_recv_count[f]       = ex[f+1] - ex[first f of e's rank]
//   recv_offsets[r]        = ex[r*L*W],   recv_offsets[W] = ex[W*E]
//   expert_token_nums[e]   = ex[(e+1)*W] - ex[e*W]            (counts, type 1)
//                          = ex[(e+1)*W] - ex[r*L*W]          (running sum, type 0)
// One workgroup: *out = counts[0] + ... + counts[n-1].
__device__ void block_sum_to(const int32_t* __restrict__ counts, int n, int32_t* __restrict__ out)
{
    __shared__ int32_t acc;
    if (threadIdx.x == 0) acc = 0;
    __syncthreads();
    int32_t c = 0;
    for (int q = threadIdx.x; q < n; q += blockDim.x) c += counts[q];
    if (c != 0) atomicAdd(&acc, c);
    __syncthreads();
    if (threadIdx.x == 0) *out = acc;
}

// One block-wide scan (each thread a run of consecutive entries, wave shuffles, LDS across
// waves), then coalesced stores.  With bad_word, also the total of the route's bad counts.
__global__ __launch_bounds__(kScanThreads) void scan_flat_kernel(
    int W, int E, int L, int etn_type, int32_t* __restrict__ seg,
    int32_t* __restrict__ ep_recv_count, int64_t* __restrict__ expert_token_nums,
    int64_t* __restrict__ recv_offsets, const int32_t* __restrict__ bad_counts,
    int32_t* __restrict__ bad_word)
{
    if (bad_word) block_sum_to(bad_counts, W, bad_word);
    // entry f is kept at LDS word f + f/32: one pad word per 32 spreads each thread's run of
    // consecutive entries over the banks (a plain layout puts a wave's runs on 4 banks)
    extern __shared__ int32_t lds_ex[];      // padded N + 1 entries, then E rank bases
    __shared__ int32_t wave_tot[kScanThreads / kWave];
    const int N = E * W;
    int32_t* rank_first = lds_ex + N + 1 + ((N + 1) >> 5) + 1;
    const int t = threadIdx.x;
#define ex(f) lds_ex[(f) + ((f) >> 5)]
    // all of this thread's counts are requested before the first is stored to LDS, so the
    // loads are in flight together (the launch has kScanThreads threads and N fits in LDS)
    int32_t staged[kScanLdsCounts / kScanThreads];
#pragma unroll
    for (int j = 0; j < kScanLdsCounts / kScanThreads; ++j) {
        const int f = t + j * kScanThreads;
        staged[j] = f < N ? seg[f] : 0;
    }
#pragma unroll
    for (int j = 0; j < kScanLdsCounts / kScanThreads; ++j) {
        const int f = t + j * kScanThreads;
        if (f < N) ex(f) = staged[j];
    }
    __syncthreads();
    const int per = (N + blockDim.x - 1) / blockDim.x;
    const int lo = min(N, t * per);
    const int hi = min(N, lo + per);
    int32_t run = 0;
    for (int f = lo; f < hi; ++f) run += ex(f);
    const int32_t incl = block_inclusive_scan(run, wave_tot);
    int32_t acc = incl - run;
    for (int f = lo; f < hi; ++f) {
        const int32_t c = ex(f);
        ex(f) = acc;
        acc += c;
    }
    if (t == blockDim.x - 1) ex(N) = incl;
    __syncthreads();
    // per expert: its rank's first entry, expert_token_nums; per rank: recv_offsets
    for (int e = t; e < E; e += blockDim.x) {
        const int first = (e / L) * L * W;
        rank_first[e] = ex(first);
        const int last = (e + 1) * W;
        const int from = etn_type == 0 ? first : e * W;
        expert_token_nums[e] = (int64_t)(ex(last) - ex(from));
    }
    for (int r = t; r <= W; r += blockDim.x) {
        const int f = r * L * W;
        recv_offsets[r] = ex(f);
    }
    __syncthreads();
    // coalesced stores over (expert, source): thread t covers source t % W of experts
    // e0 + t / W, e0 advancing by rows = blockDim / W per pass (one division per thread)
    const int rows = blockDim.x / W;
    const int te = t / W;
    const int ts = t - te * W;
    if (te < rows) {
        for (int e = te; e < E; e += rows) {
            const int f = e * W + ts;
            const int f1 = f + 1;
            seg[f] = ex(f);
            ep_recv_count[f] = ex(f1) - rank_first[e];
        }
    }
#undef ex
}

// One workgroup: *out = the sum of every thread's v.
__device__ void block_sum_to_value(int32_t v, int32_t* __restrict__ out)
{
    __shared__ int32_t acc;
    if (threadIdx.x == 0) acc = 0;
    __syncthreads();
    if (v != 0) atomicAdd(&acc, v);
    __syncthreads();
    if (threadIdx.x == 0) *out = acc;
}

// Receive-side scan for shapes whose counts exceed one workgroup's LDS budget (E*W >
// kScanMaxFlat), in two launches over groups of whole receiver ranks.  Every output of a
// rank r -- its ep_recv_count row, its experts' expert_token_nums, recv_offsets[r] -- is a
// difference of running totals inside the rank's own entries [r*L*W, (r+1)*L*W), except for
// one offset common to all of them: the number of rows of the ranks before it.  So the ranks
// are cut into groups of R consecutive ranks (R*L*W <= kGroupCounts; one rank has
// L*W <= 2048 entries, so R >= 7); scan_group_totals_kernel sums each group's counts, and
// scan_groups_kernel adds up the totals of the groups before its own and then scans its
// group in LDS exactly as scan_flat_kernel scans the whole array.
__global__ __launch_bounds__(kScanThreads) void scan_group_totals_kernel(
    int W, int L, int R, const int32_t* __restrict__ seg, int32_t* __restrict__ totals,
    const int32_t* __restrict__ bad_counts, int32_t* __restrict__ bad_word)
{
    if (blockIdx.x == 0 && bad_word) block_sum_to(bad_counts, W, bad_word);
    const int LW = L * W;
    const int r0 = blockIdx.x * R;
    const int r1 = min(W, r0 + R);
    const int f0 = r0 * LW;
    const int n = (r1 - r0) * LW;
    int32_t c[kScanLdsCounts / kScanThreads];
#pragma unroll
    for (int j = 0; j < kScanLdsCounts / kScanThreads; ++j) {
        const int f = threadIdx.x + j * kScanThreads;
        c[j] = f < n ? seg[f0 + f] : 0;
    }
    int32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kScanLdsCounts / kScanThreads; ++j) sum += c[j];
    block_sum_to_value(sum, &totals[blockIdx.x]);
}

__global__ __launch_bounds__(kScanThreads) void scan_groups_kernel(
    int W, int E, int L, int R, int etn_type, int32_t* __restrict__ seg,
    int32_t* __restrict__ ep_recv_count, int64_t* __restrict__ expert_token_nums,
    int64_t* __restrict__ recv_offsets, const int32_t* __restrict__ totals)
{
    extern __shared__ int32_t lds_grp[];     // padded group entries + 1
    __shared__ int32_t wave_tot[kScanThreads / kWave];
    __shared__ int32_t before_lds;
    const int LW = L * W;
    const int g = blockIdx.x;
    const int r0 = g * R;
    const int r1 = min(W, r0 + R);
    const int f0 = r0 * LW;
    const int n = (r1 - r0) * LW;
    const int t = threadIdx.x;
    const int nt = blockDim.x;
#define ex(f) lds_grp[(f) + ((f) >> 5)]
    // this group's counts, requested together with the earlier groups' totals
    int32_t staged[kScanLdsCounts / kScanThreads];
#pragma unroll
    for (int j = 0; j < kScanLdsCounts / kScanThreads; ++j) {
        const int f = t + j * kScanThreads;
        staged[j] = f < n ? seg[f0 + f] : 0;
    }
    int32_t prior = 0;
    for (int q = t; q < g; q += nt) prior += totals[q];
    if (t == 0) before_lds = 0;
#pragma unroll
    for (int j = 0; j < kScanLdsCounts / kScanThreads; ++j) {
        const int f = t + j * kScanThreads;
        if (f < n) ex(f) = staged[j];
    }
    __syncthreads();
    if (prior != 0) atomicAdd(&before_lds, prior);
    const int per = (n + nt - 1) / nt;
    const int lo = min(n, t * per);
    const int hi = min(n, lo + per);
    int32_t run = 0;
    for (int f = lo; f < hi; ++f) run += ex(f);
    const int32_t incl = block_inclusive_scan(run, wave_tot);   // its barrier also publishes
    const int32_t before = before_lds;                           // before_lds
    int32_t acc = before + incl - run;
    for (int f = lo; f < hi; ++f) {
        const int32_t c = ex(f);
        ex(f) = acc;
        acc += c;
    }
    if (t == nt - 1) ex(n) = before + incl;
    __syncthreads();
    for (int f = t; f < n; f += nt) {
        seg[f0 + f] = ex(f);
        const int rank_first = (f / LW) * LW;
        ep_recv_count[f0 + f] = ex(f + 1) - ex(rank_first);
    }
    for (int e = r0 * L + t; e < r1 * L; e += nt) {
        const int rank_first = (e / L) * LW - f0;
        const int from = etn_type == 0 ? rank_first : e * W - f0;
        expert_token_nums[e] = (int64_t)(ex((e + 1) * W - f0) - ex(from));
    }
    for (int r = r0 + t; r < r1; r += nt) recv_offsets[r] = ex(r * LW - f0);
    if (r1 == W && t == 0) recv_offsets[W] = ex(n);
#undef ex
}

}  // namespace

hipError_t launch_route(const Shape& sh, const int32_t* expert_ids, const uint8_t* mask,
                        int32_t* expand_idx, int32_t* seg, int32_t* bad_counts,
                        hipStream_t stream)
{
    // about one workgroup per CU: (W source ranks) x (groups of experts)
    const int nwords = (sh.BS + 31) / 32;
    int groups = 256 / sh.W;
    const int max_groups = (sh.E + 15) / 16;
    groups = groups < 1 ? 1 : (groups > max_groups ? max_groups : groups);
    int group = (sh.E + groups - 1) / groups;
    if (group > kMaxRouteExperts) group = kMaxRouteExperts;
    groups = (sh.E + group - 1) / group;
    const size_t lds = (size_t)4 * group * nwords * sizeof(uint32_t);
    const int threads = (sh.BS + kWave - 1) / kWave * kWave;      // one lane per token
    const dim3 grid(sh.W, groups);
    const bool vec = (sh.K % 4 == 0) && ((reinterpret_cast<uintptr_t>(expert_ids) & 15) == 0);
#define MOE_DC_ROUTE(KM, V)                                                                      \
    hipLaunchKernelGGL((route_kernel<KM, V>), grid, dim3(threads), lds, stream, expert_ids,     \
                       mask, sh.mask_kind, sh.W, sh.E, sh.BS, sh.K, nwords, group, expand_idx, \
                       seg, bad_counts, sh.id_end)
    if (sh.K <= 2) MOE_DC_ROUTE(2, false);
    else if (sh.K <= 4) { if (vec && sh.K == 4) MOE_DC_ROUTE(4, true); else MOE_DC_ROUTE(4, false); }
    else if (sh.K <= 8) { if (vec && sh.K == 8) MOE_DC_ROUTE(8, true); else MOE_DC_ROUTE(8, false); }
    else { if (vec && sh.K == 16) MOE_DC_ROUTE(16, true); else MOE_DC_ROUTE(16, false); }
#undef MOE_DC_ROUTE
    return hipGetLastError();
}

hipError_t launch_scan(const Shape& sh, int32_t* seg, int32_t* ep_recv_count,
                       int64_t* expert_token_nums, int64_t* recv_offsets,
                       const int32_t* bad_counts, int32_t* bad_word, int32_t* totals,
                       hipStream_t stream)
{
    const long long n = (long long)sh.E * sh.W;
    if (n <= kScanMaxFlat) {
        const size_t words = (size_t)n + 1 + (size_t)((n + 1) >> 5) + 1 + sh.E;
        hipLaunchKernelGGL(scan_flat_kernel, dim3(1), dim3(kScanThreads),
                           words * sizeof(int32_t), stream, sh.W, sh.E, sh.L, sh.etn_type, seg,
                           ep_recv_count, expert_token_nums, recv_offsets, bad_counts, bad_word);
    } else {
        // groups of R whole ranks, R * L * W <= kGroupCounts (L * W <= 2048 gives R >= 7)
        const int LW = sh.L * sh.W;
        const int R = kGroupCounts / LW;
        const int G = (sh.W + R - 1) / R;
        const size_t words = (size_t)R * LW + 1 + (((size_t)R * LW + 1) >> 5) + 1;
        hipLaunchKernelGGL(scan_group_totals_kernel, dim3(G), dim3(kScanThreads), 0, stream,
                           sh.W, sh.L, R, seg, totals, bad_counts, bad_word);
        hipLaunchKernelGGL(scan_groups_kernel, dim3(G), dim3(kScanThreads),
                           words * sizeof(int32_t), stream, sh.W, sh.E, sh.L, R, sh.etn_type,
                           seg, ep_recv_count, expert_token_nums, recv_offsets, totals);
    }
    return hipGetLastError();
}

}  // namespace moe_dc
