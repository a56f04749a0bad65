// dispatch.hip -- quantize each source token and write it to its K packed rows.
//
// Vectorized path (H % 8 == 0, 16-byte aligned pointers): one workgroup per source token
// (s, i); each wavefront owns two slots of 64 16-byte vectors (8 bf16 elements per lane, so
// every load instruction covers 1 KiB of contiguous memory).  All waves issue their row
// loads first; threads 0..K-1 resolve the token's K destination rows meanwhile; one barrier
// publishes the rows (and, for per-token scaling, the per-wave maxima of the token).  Each
// wave then quantizes its slots in registers and stores them to the final row of every
// routed pick.  Rows are read and written with the non-temporal cache policy (each is
// touched exactly once).  Small workgroups, many of them, keep every SIMD busy until the end
// of the launch.
//
// Destination rows follow the pages' placement rule (design doc §2.2.2 token reorder and
// §2.4 post-processing, merged into one address because every receiver lives in this GPU's
// memory): the (expert, source) segment base left in the workspace by the scan kernel plus
// the pick's expand_idx.
//
// Quantization (low_latency_dispatch, 计算公式 and 约束说明; ops-transformer article,
// 功能说明 情形 2).  x_fp32 is the bf16 token widened, times the scales tensor when one is
// given: a scalar, a row shared by every expert, or the routed expert's row of an [E][H]
// table (then the codes differ per pick and each pick is quantized on its own).
//   mode 0  rows copied bit for bit
//   mode 1  codes = int8(x_fp32): static scales, no scales out
//   mode 2  dyn = type_max / max|x_fp32| over the token, codes = type(x_fp32 * dyn),
//           scale = 1 / dyn (type int8, E4M3 or E5M2; max 127, 448, 57344)
//   mode 3  as mode 2 over each group of 128 elements; Ceil(H, 128) scales per row
//   mode 4  per 32-element block: shared_exp = floor(log2 max|x|) - emax (clamped at -127;
//           emax 8 for E4M3, 15 for E5M2)
//   mode 5  per block: shared_exp = ceil(log2(max(max|x|, 1e-4) / fp8_max))
//           codes = fp8(x / 2^shared_exp); the scale written is 2^shared_exp, as fp32 or as
//           its E8M0 byte shared_exp + 127 (the SMP article's stored format), or, as the
//           low_latency_dispatch formula writes it, its reciprocal 2^-shared_exp in fp32
//           (exact: shared_exp lies in [-127, 126]).  Modes 4/5 also take E2M1 (fp4: emax
//           2, max 6) elements, two 4-bit codes per byte with the even element in the low
//           nibble.
// int8 rounds half to even and saturates at +-127 with NaN -> 0; fp8 rounds to nearest even
// and saturates at the type's largest finite value; NaN products of a dynamic mode (only
// 0 * inf of an all-zero segment) give code 0.  In the vectorized path an MX block is 4
// adjacent lanes and a group of 128 is 16 adjacent lanes, reduced with lane exchanges.
//
// Per-expert scales ([E][H]: a pick's codes depend on its expert) have two more layouts in
// the vectorized path, chosen by batch size: one small workgroup per pick for small batches
// (scatter_pick_kernel), and for large ones one workgroup per (window of tokens, expert)
// that keeps the expert's scales row in registers (scatter_window_kernel).  Batches that
// route inside the scatter launch use the token workgroups.
//
// The element-wise fallback (any H, any alignment) uses one workgroup per token with one
// element per lane (scatter_elem_kernel); the variant is a runtime argument there.
#include "dc_device.h"
#include "dc_convert.h"
#include "route_device.h"
#include "dc_internal.h"

namespace moe_dc {
namespace {

constexpr int kGroup = 128;          // mode 3 group length


template <int CT>
__device__ __forceinline__ uint32_t fp8_code(float v)
{
    return CT == kCodeE4m3 ? e4m3_code(v) : CT == kCodeE5m2 ? e5m2_code(v) : e2m1_code(v);
}

// Largest finite value of a code type (dst_type_max / fp8_max of the formulas).
template <int CT>
constexpr float type_max()
{
    return CT == kCodeInt8 ? 127.0f : CT == kCodeE4m3 ? 448.0f : CT == kCodeE5m2 ? 57344.0f
                                                                                 : 6.0f;
}

// A per-128-group dynamic scale pair (mode 3): dyn = type_max / amax and scale = 1 / dyn, both
// correctly rounded, as the per-element division gives them.
template <int CT>
__device__ __forceinline__ void group_dyn(uint32_t amax_bits, float& dyn, float& scale)
{
    const float amax = __uint_as_float(amax_bits);
    if (CT == kCodeE4m3) dyn = div_rn<8>(448.0f, amax);
    else if (CT == kCodeE5m2) dyn = div_rn<15>(57344.0f, amax);
    else dyn = type_max<CT>() / amax;
    scale = div_rn<1>(1.0f, dyn);
}

// Shared exponent of an MX block from the bit pattern of its absolute maximum.
template <int MODE, int CT>
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits)
{
    constexpr int emax = CT == kCodeE4m3 ? 8 : CT == kCodeE5m2 ? 15 : 2;
    if (MODE == 4) {
        if (amax_bits == 0) return -127;
        const int ex = (int)(amax_bits >> 23);
        const int fl = ex != 0 ? ex - 127 : (31 - __clz(amax_bits)) - 149;   // floor(log2)
        return fl - emax > -127 ? fl - emax : -127;
    } else {
        const float c = fmaxf(__uint_as_float(amax_bits), 1e-4f);
        const uint32_t vb = __float_as_uint(c / type_max<CT>());           // normal, > 0
        return (int)(vb >> 23) - 127 + ((vb & 0x7FFFFFu) != 0u ? 1 : 0);     // ceil(log2)
    }
}

// 2^e for e in [-127, 126] as a binary32 (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2f(int e)
{
    return e >= -126 ? __uint_as_float((uint32_t)(127 + e) << 23) : __uint_as_float(0x00400000u);
}

// Eight token elements of one 16-byte vector, widened to binary32 (exact): bf16, or
// binary16 when f16 is set (a wave-uniform flag).
__device__ __forceinline__ void unpack8(uint4 w, float (&f)[8], bool f16)
{
    if (f16) {
        f[0] = f16_lo(w.x); f[1] = f16_hi(w.x); f[2] = f16_lo(w.y); f[3] = f16_hi(w.y);
        f[4] = f16_lo(w.z); f[5] = f16_hi(w.z); f[6] = f16_lo(w.w); f[7] = f16_hi(w.w);
    } else {
        f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
        f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
    }
}

__device__ __forceinline__ void mul8(float (&f)[8], float4 a, float4 b)
{
    f[0] = f[0] * a.x; f[1] = f[1] * a.y; f[2] = f[2] * a.z; f[3] = f[3] * a.w;
    f[4] = f[4] * b.x; f[5] = f[5] * b.y; f[6] = f[6] * b.z; f[7] = f[7] * b.w;
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

// absmax8 for values that are products of a multiplication (canonical floats, never NaN for
// finite inputs): a float maximum of absolute values, which the compiler forms from max3
// instructions with absolute-value operand modifiers; for non-negative non-NaN floats the
// float order is the order of the bit patterns, so the result is absmax8's.
__device__ __forceinline__ uint32_t absmax8_products(const float (&f)[8], uint32_t amax)
{
    float m = __uint_as_float(amax);
#pragma unroll
    for (int c = 0; c < 8; ++c) m = __builtin_fmaxf(m, __builtin_fabsf(f[c]));
    return __float_as_uint(m);
}

__device__ __forceinline__ uint2 pack_codes8(const uint32_t (&c)[8])
{
    return make_uint2((c[0] & 0xFF) | ((c[1] & 0xFF) << 8) | ((c[2] & 0xFF) << 16) | (c[3] << 24),
                      (c[4] & 0xFF) | ((c[5] & 0xFF) << 8) | ((c[6] & 0xFF) << 16) | (c[7] << 24));
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

// Eight codes of the dynamic modes: type(f * dyn), NaN products -> 0.
template <int CT>
__device__ __forceinline__ uint2 dynamic_codes8(const float (&f)[8], float dyn)
{
    if (CT == kCodeInt8 && __float_as_uint(dyn) < 0x7F800000u)    // dyn > 0 here
        return int8_codes8_finite(f, dyn);
    if (CT == kCodeE4m3 || CT == kCodeE5m2) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float p = f[q] * dyn;
            v[q] = p != p ? 0.0f : p;                  // a NaN product's code is 0
        }
        return fp8_codes8_hw<CT>(v);
    }
    uint32_t c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float v = f[q] * dyn;
        if (CT == kCodeInt8) c[q] = int8_code(v);
        else c[q] = v != v ? 0u : fp8_code<CT>(v);
    }
    return pack_codes8(c);
}

// Eight static int8 codes (mode 1): the scales are already applied.
__device__ __forceinline__ uint2 static_codes8(const float (&f)[8])
{
    return static_int8_codes8(f);
}

// ---------------------------------------------------------------------------------------
// vectorized path: one workgroup per token, kTileSlots 64-vector slots per wave
// ---------------------------------------------------------------------------------------

constexpr int kTileSlots = 2;        // 64-vector slots (1 KiB of bf16 each) per wave
constexpr int kMaxTileWaves = 8;     // H <= 8192: at most 1024 vectors = 16 slots
constexpr int kFusedMinWaves = 4;    // workgroup size floor when the launch also routes

// Per-wave maxima meet in LDS slots, one per wave, read back as a fixed, unrolled set of
// kMaxTileWaves slots (a loop over the workgroup's wave count waited for each read in turn).
// The slots of waves the workgroup does not have are cleared first; no wave writes them.
__device__ __forceinline__ void clear_spare_slots(uint32_t (&red)[2][kMaxTileWaves], int nw)
{
    const int t = threadIdx.x;
    if (t < 2 * kMaxTileWaves && t % kMaxTileWaves >= nw)
        red[t / kMaxTileWaves][t % kMaxTileWaves] = 0u;
}

__device__ __forceinline__ uint32_t slots_max(const uint32_t (&slots)[kMaxTileWaves])
{
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < kMaxTileWaves; ++w) m = m > slots[w] ? m : slots[w];
    return m;
}

// Small batches route inside the scatter launch (all picks fit in one pass of a workgroup).
// Workgroup 0 produces the receive-side outputs; every other workgroup finds the packed rows
// of its own token's picks by counting.  Counting commutes, so no result depends on the
// order in which atomics land.

// Workgroup 0: routed-pick counts per (expert e, source rank s') at ex[e*W + s'] in LDS,
// their exclusive running total over that flat order (ex[E*W] = all routed rows), and from
// it ep_recv_count, expert_token_nums and recv_offsets -- what the route and scan kernels
// write for larger batches.  With fr.bad_word, also the number of active picks whose id
// lies outside [0, fr.id_end).
__device__ void route_totals(const int32_t* __restrict__ ids, const FusedRoute& fr, int W,
                             int E, int L, int BS, int K, int mask_kind, int etn_type,
                             int32_t* ex, int32_t* wave_tot)
{
    const int t = threadIdx.x;
    const int nt = blockDim.x;
    const int N = E * W;
    const int picks = W * BS * K;
    __shared__ int32_t bad_lds;
    for (int f = t; f < N; f += nt) ex[f] = 0;
    if (t == 0) bad_lds = 0;
    __syncthreads();
    int32_t bad = 0;
    for (int p = t; p < picks; p += nt) {
        const int q = p / K;
        const int32_t e = routed_expert(ids, fr.mask, mask_kind, K, E, q, p - q * K);
        if (e >= 0) atomicAdd(&ex[e * W + q / BS], 1);
        if (fr.bad_word) bad += bad_pick(ids, fr.mask, mask_kind, K, fr.id_end, q, p - q * K);
    }
    if (bad != 0) atomicAdd(&bad_lds, bad);
    __syncthreads();
    if (fr.bad_word && t == 0) *fr.bad_word = bad_lds;
    // exclusive running total in place: each thread scans one run of entries
    const int per = (N + nt - 1) / nt;
    const int lo = min(N, t * per);
    const int hi = min(N, lo + per);
    int32_t run = 0;
    for (int f = lo; f < hi; ++f) run += ex[f];
    const int32_t incl = block_inclusive_scan(run, wave_tot);
    int32_t acc = incl - run;
    for (int f = lo; f < hi; ++f) {
        const int32_t cnt = ex[f];
        ex[f] = acc;
        acc += cnt;
    }
    if (t == nt - 1) ex[N] = incl;
    __syncthreads();
    // receiver r = e / L: ep_recv_count runs from the rank's first segment; recv_offsets[r]
    // is the rank's first row; expert_token_nums counts per expert (type 1) or runs (type 0)
    for (int f = t; f < N; f += nt)
        fr.ep_recv_count[f] = ex[f + 1] - ex[(f / W / L) * L * W];
    for (int e = t; e < E; e += nt) {
        const int first = (e / L) * L * W;
        const int from = etn_type == 0 ? first : e * W;
        fr.expert_token_nums[e] = (int64_t)(ex[(e + 1) * W] - ex[from]);
    }
    for (int r = t; r <= W; r += nt) fr.recv_offsets[r] = ex[r * L * W];
}

// Picks each thread of a token workgroup counts: t, t + blockDim, ... (blockDim >= 256).
constexpr int kFusedPicksPerThread = (int)(kFusedMaxPicks / (kWave * kFusedMinWaves));

// The routed expert (or -1) of each pick this thread counts, and in lane k < K of every
// wave that of the workgroup's own pick k.  Called before the token row is requested: loads
// complete in issue order, so using these values then does not wait for the row.
__device__ __forceinline__ int32_t load_fused_picks(const int32_t* __restrict__ ids,
                                                    const FusedRoute& fr, int E, int K,
                                                    int mask_kind, int picks, long long tok,
                                                    int32_t (&pe)[kFusedPicksPerThread])
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t own_e =
        lane < K ? routed_expert(ids, fr.mask, mask_kind, K, E, tok, lane) : -1;
#pragma unroll
    for (int j = 0; j < kFusedPicksPerThread; ++j) {
        const int p2 = threadIdx.x + j * blockDim.x;
        pe[j] = -1;
        if (p2 < picks) {
            const int q = p2 / K;
            pe[j] = routed_expert(ids, fr.mask, mask_kind, K, E, q, p2 - q * K);
        }
    }
    return own_e;
}

// Token workgroups: the packed row of pick k of token `tok` (source rank s) is its position in
// the stable sort of all routed picks by (expert, source rank, token, pick), i.e. the number
// of routed picks p2 with a smaller expert, or the same expert and p2 < tok*K + k in the
// flat (rank, token, pick) order.  Its expand_idx counts only the same expert's picks of
// rank s before it.  Threads k < K get the row of pick k (-1 when it is not routed, or past
// `cap`) and write its expand_idx.  Both counts of a pick share one word (16 bits each; a
// batch has at most kFusedMaxPicks picks); the words are summed across each wave with the
// device library's data-parallel-primitive reduction, then across waves by LDS atomics.
__device__ int32_t route_own_rows(int K, int BS, int tok, int s, long long cap,
                                  const int32_t (&pe)[kFusedPicksPerThread], int32_t own_e,
                                  int32_t* row_lds, int32_t* ord_lds,
                                  int32_t* __restrict__ expand_idx)
{
    const int t = threadIdx.x;
    const int nt = blockDim.x;
    const int own = tok * K;
    const int rank_lo = s * BS * K;
    if (t < kMaxK) {
        row_lds[t] = 0;
        ord_lds[t] = 0;
    }
    int32_t mine[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) mine[k] = lane_value(own_e, k);   // -1 for k >= K
    uint32_t cnt[kMaxK];                  // before | same << 16
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) cnt[k] = 0;
#pragma unroll
    for (int j = 0; j < kFusedPicksPerThread; ++j) {
        const int p2 = t + j * nt;
        const int32_t e2 = pe[j];
        if (e2 < 0) continue;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            const bool earlier = e2 == mine[k] && p2 < own + k;
            cnt[k] += (e2 < mine[k] || earlier) ? 1u : 0u;
            cnt[k] += (earlier && p2 >= rank_lo) ? 0x10000u : 0u;
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) cnt[k] = __ockl_wfred_add_u32(cnt[k]);   // wave sums (DPP)
    __syncthreads();                                      // row_lds / ord_lds cleared
    if ((t & (kWave - 1)) == 0) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            const int32_t before = (int32_t)(cnt[k] & 0xFFFFu);
            const int32_t same = (int32_t)(cnt[k] >> 16);
            if (k < K && before != 0) atomicAdd(&row_lds[k], before);
            if (k < K && same != 0) atomicAdd(&ord_lds[k], same);
        }
    }
    __syncthreads();
    int32_t row = -1;
    if (t < K) {
        const bool routed = own_e >= 0;                   // lane t of wave 0: own pick t
        expand_idx[own + t] = routed ? ord_lds[t] : -1;
        if (routed && row_lds[t] < cap) row = row_lds[t];
    }
    return row;
}

// MODE 0..5, CT the code type, SK the scales kind.  FUSED: the launch also routes, with one
// extra workgroup (0, route_totals; E*W + 1 words of dynamic LDS) before the token
// workgroups (route_own_rows); a separate instantiation, so the large-batch kernels keep
// their register budget.
template <int MODE, int CT, int SK, bool FUSED>
__global__ __launch_bounds__(kWave * kMaxTileWaves) void scatter_tile_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    int32_t* __restrict__ expand_idx, const int32_t* __restrict__ seg,
    const float* __restrict__ scales, const float* __restrict__ weights,
    void* __restrict__ expand_x, void* __restrict__ dyn_scales, int32_t* __restrict__ assist,
    float* __restrict__ expand_scales, int W, int E, int BS, int H, int K, int ns,
    long long cap, int sfmt, FusedRoute fr, int L, int mask_kind, int etn_type, int tok_f16)
{
    __shared__ int32_t rows_lds[kMaxK];
    __shared__ int32_t exps_lds[kMaxK];
    __shared__ int32_t pick_row_lds[kMaxK];   // per-expert scales: the routed picks' rows
    __shared__ int32_t pick_exp_lds[kMaxK];   // and experts, in k order
    __shared__ uint32_t red[2][kMaxTileWaves];
    __shared__ int32_t ord_lds[kMaxK];
    __shared__ int32_t fused_rows_lds[kMaxK];
    __shared__ int32_t wave_tot[kMaxTileWaves];
    extern __shared__ int32_t route_ex[];

    if (FUSED && blockIdx.x == 0) {
        route_totals(ids, fr, W, E, L, BS, K, mask_kind, etn_type, route_ex, wave_tot);
        return;
    }

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const long long tok = FUSED ? blockIdx.x - 1 : blockIdx.x;
    clear_spare_slots(red, nw);
    const int s = (int)(tok / BS);
    const int i = (int)(tok - (long long)s * BS);
    const int NV = H >> 3;
    float* fscales = static_cast<float*>(dyn_scales);

    int32_t fused_picks[kFusedPicksPerThread];
    int32_t fused_own = -1;
    if (FUSED) fused_own = load_fused_picks(ids, fr, E, K, mask_kind, W * BS * K, tok, fused_picks);

    // Under a mask a token may have no routed pick at all: then its row is never needed, so
    // the token's expand_idx entries (written by the route kernel) are read first and such a
    // token leaves before requesting its row.  Unmasked batches skip this wait.
    if (!FUSED && mask_kind != 0) {
        const int32_t ord = lane < K ? expand_idx[tok * K + lane] : -1;
        if (__ballot(ord >= 0) == 0) return;              // uniform over the workgroup
    }

    // 1. this wave's slots of the token row (and of a shared scales row), in flight before
    //    anything waits
    const uint4* xr = reinterpret_cast<const uint4*>(x) + tok * NV;
    uint4 raw[kTileSlots];
    float4 shared_pre[kTileSlots][2];
#pragma unroll
    for (int n = 0; n < kTileSlots; ++n) {
        const int v = lane + (wave * kTileSlots + n) * kWave;
        raw[n] = make_uint4(0u, 0u, 0u, 0u);
        if (v < NV) {
            raw[n] = load_stream(xr + v);
            if (SK == kScalesShared) {
                const float4* sm = reinterpret_cast<const float4*>(scales);
                shared_pre[n][0] = sm[2 * v];
                shared_pre[n][1] = sm[2 * v + 1];
            }
        }
    }
    const float scalar_pre = SK == kScalesScalar ? scales[0] : 1.0f;

    // 2. destination rows, resolved by threads 0..K-1 (small batches route here first)
    int32_t fused_row = -1;
    if (FUSED)
        fused_row = route_own_rows(K, BS, (int)tok, s, cap, fused_picks, fused_own,
                                   fused_rows_lds, ord_lds, expand_idx);
    if (threadIdx.x < K) {
        const long long p = tok * K + threadIdx.x;
        const int32_t e = ids[p];
        int32_t row = -1;
        if (FUSED) {
            row = fused_row;
        } else {
            const int32_t ord = expand_idx[p];
            if (ord >= 0 && e >= 0 && e < E) {
                const long long r = (long long)seg[(long long)e * W + s] + ord;
                if (r < cap) row = (int32_t)r;
            }
        }
        rows_lds[threadIdx.x] = row;
        exps_lds[threadIdx.x] = e;
        if (SK == kScalesPerExpert) {
            // threads 0..K-1 are lanes of wave 0: a routed pick's place in the list is the
            // number of routed picks before it
            const uint64_t routed = __ballot(row >= 0);
            if (row >= 0) {
                const int j = __popcll(routed & ((1ull << threadIdx.x) - 1ull));
                pick_row_lds[j] = row;
                pick_exp_lds[j] = e;
            }
        }
        if (row >= 0) {
            assist[(long long)row * 3 + 0] = s;
            assist[(long long)row * 3 + 1] = i;
            assist[(long long)row * 3 + 2] = threadIdx.x;
            if (expand_scales) expand_scales[row] = weights[p];
        }
    }

    // x_fp32 of this wave's slots when the codes are shared by every pick
    float f[kTileSlots][8];
    if (MODE != 0 && SK != kScalesPerExpert) {
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = lane + (wave * kTileSlots + n) * kWave;
            if (v < NV) {
                unpack8(raw[n], f[n], tok_f16 != 0);
                if (SK == kScalesScalar) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) f[n][q] = f[n][q] * scalar_pre;
                }
                if (SK == kScalesShared) mul8(f[n], shared_pre[n][0], shared_pre[n][1]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) f[n][q] = 0.0f;
            }
        }
    }

    // 3. the token's absolute maximum (mode 2 with shared codes), per wave first
    if (MODE == 2 && SK != kScalesPerExpert) {
        uint32_t amax = 0;
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) amax = absmax8(f[n], amax);
        amax = wave_max_u32(amax);
        if (lane == 0) red[0][wave] = amax;
    }
    __syncthreads();

    int rows[kMaxK];
    int n_routed = 0;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        rows[k] = k < K ? __builtin_amdgcn_readfirstlane(rows_lds[k]) : -1;
        n_routed += rows[k] >= 0 ? 1 : 0;
    }
    if (n_routed == 0) return;                             // uniform over the workgroup

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

    if (SK != kScalesPerExpert) {
        // codes shared by every pick: quantize once, store K times
        float dyn_tok = 0.0f;
        if (MODE == 2) {
            dyn_tok = type_max<CT>() / __uint_as_float(slots_max(red[0]));
        }
        uint32_t fp4_words[kTileSlots];     // E2M1: this lane's eight codes, per slot
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = lane + (wave * kTileSlots + n) * kWave;
            uint2 packed;
            float scale = 0.0f;             // per group (mode 3) or per block (modes 4/5)
            int se = 0;
            if (MODE == 1) {
                packed = static_codes8(f[n]);
            } else if (MODE == 2) {
                packed = dynamic_codes8<CT>(f[n], dyn_tok);
            } else if (MODE == 3) {
                const uint32_t amax = group_max_u32<kGroup / 8>(absmax8(f[n], 0u));
                float dyn;
                group_dyn<CT>(amax, dyn, scale);
                packed = dynamic_codes8<CT>(f[n], dyn);
            } else {
                const uint32_t amax = group_max_u32<kMxBlock / 8>(absmax8(f[n], 0u));
                se = mx_shared_exp<MODE, CT>(amax);
                const float inv = __uint_as_float((uint32_t)(127 - se) << 23);   // 2^-se
                // a NaN element saturates with its sign, as fp8_code gives it
                float e[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float p = f[n][q] * inv;
                    e[q] = p != p ? __builtin_copysignf(type_max<CT>(), p) : p;
                }
                if (CT == kCodeE2m1) {            // eight 4-bit codes, element 0 lowest
                    const uint32_t w = fp4_word_hw(e);
                    fp4_words[n] = w;
                    packed = make_uint2(w, 0u);
                } else {
                    packed = fp8_codes8_hw<CT>(e);
                }
                scale = sfmt == 2 ? inv : pow2f(se);      // 1 / 2^se, or 2^se
            }
            if (v >= NV) continue;
#pragma unroll
            for (int k = 0; k < kMaxK; ++k) {
                if (rows[k] < 0) continue;
                if (CT == kCodeE2m1) {
                    if (NV & 1)                   // odd vector count: 4-byte stores
                        __builtin_nontemporal_store(
                            packed.x,
                            reinterpret_cast<uint32_t*>(expand_x) + (long long)rows[k] * NV + v);
                } else {
                    store_stream(out + (long long)rows[k] * NV + v, packed);
                }
                if (MODE == 3 && (v & (kGroup / 8 - 1)) == 0)
                    fscales[(long long)rows[k] * ns + (v >> 4)] = scale;
                if (MODE >= 4 && (v & 3) == 0) {
                    if (sfmt == 1)
                        static_cast<uint8_t*>(dyn_scales)[(long long)rows[k] * ns + (v >> 2)] =
                            (uint8_t)(se + 127);
                    else
                        fscales[(long long)rows[k] * ns + (v >> 2)] = scale;
                }
            }
        }
        if (CT == kCodeE2m1 && (NV & 1) == 0) {
            // The wave's two slots hold vectors [wave * 128, wave * 128 + 128); lane l writes
            // vectors 2l and 2l + 1 (from slot l / 32) as one 8-byte store, so each store
            // instruction covers 512 contiguous bytes.
            const int src = (2 * lane) & (kWave - 1);
            const uint32_t a0 = __shfl(fp4_words[0], src, kWave);
            const uint32_t b0 = __shfl(fp4_words[0], src + 1, kWave);
            const uint32_t a1 = __shfl(fp4_words[1], src, kWave);
            const uint32_t b1 = __shfl(fp4_words[1], src + 1, kWave);
            const uint2 pair = lane < kWave / 2 ? make_uint2(a0, b0) : make_uint2(a1, b1);
            const int vpair = wave * kTileSlots * kWave + 2 * lane;
            if (vpair < NV) {
#pragma unroll
                for (int k = 0; k < kMaxK; ++k)
                    if (rows[k] >= 0)
                        store_stream(out + ((long long)rows[k] * NV + vpair) / 2, pair);
            }
        }
        if (MODE == 2 && threadIdx.x == 0) {
            const float scale = 1.0f / dyn_tok;
#pragma unroll
            for (int k = 0; k < kMaxK; ++k)
                if (rows[k] >= 0) fscales[rows[k]] = scale;
        }
        if (MODE >= 4 && threadIdx.x == 0) {
            const int nb = (H + kMxBlock - 1) / kMxBlock;
            if (ns > nb) {
#pragma unroll
                for (int k = 0; k < kMaxK; ++k) {
                    if (rows[k] < 0) continue;
                    if (sfmt == 1) static_cast<uint8_t*>(dyn_scales)[(long long)rows[k] * ns + nb] = 0;
                    else fscales[(long long)rows[k] * ns + nb] = 0.0f;
                }
            }
        }
        return;
    }

    // Per-expert scales (modes 1-3): one quantization per pick, on its expert's row.  The
    // routed picks (listed in k order in LDS) run one after another; the scales slice of the
    // next one is loaded into the other register buffer while the current pick is quantized
    // and stored, so its latency is hidden.  The loop is unrolled by two, so the two buffers
    // alternate without copies.  The scales slices are read and the codes written through
    // range-checked buffer resources over the pick's rows, with no branch around them, so
    // waiting for a slice does not also wait for the stores issued after it; past the row's
    // end the token values and the slices read 0, so the products there are 0 and no maximum
    // needs a bounds test.  Mode 2 needs a workgroup-wide maximum per pick; modes 1 and 3 do
    // not synchronize at all.
    float xf[kTileSlots][8];
#pragma unroll
    for (int n = 0; n < kTileSlots; ++n) unpack8(raw[n], xf[n], tok_f16 != 0);
    float4 sa[kTileSlots][2], sb[kTileSlots][2];
    // vector v = lane + slot0 + 64 n of the row for slot n of this wave
    const uint32_t slot0 = (uint32_t)__builtin_amdgcn_readfirstlane(wave * kTileSlots * kWave);
    const uint32_t v0 = (uint32_t)lane + slot0;
    // past the end of the list the resource is empty: the loads return 0 and read nothing
    auto load_pre = [&](int j, float4 (&dst)[kTileSlots][2]) {
        const bool in = j < n_routed;                      // uniform
        const int e = __builtin_amdgcn_readfirstlane(pick_exp_lds[in ? j : 0]);
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales + (long long)e * H, in ? 4u * H : 0u);
        // an opaque copy of the lane offset, so the constant parts below stay with each load
        // (and go to its immediate offset) instead of each becoming a register of its own
        uint32_t off = 32u * v0;
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            dst[n][0] = rsrc_load_f4(sr, off + 2048u * n);
            dst[n][1] = rsrc_load_f4(sr, off + 2048u * n + 16u);
        }
    };
    auto quant_pick = [&](int j, const float4 (&sm)[kTileSlots][2], int buf) {
        const int prow = __builtin_amdgcn_readfirstlane(pick_row_lds[j]);
        const __amdgpu_buffer_rsrc_t orow = make_rsrc(out + (long long)prow * NV, 8u * NV);
        const __amdgpu_buffer_rsrc_t srow =
            make_rsrc(fscales + (long long)prow * ns, 4u * (uint32_t)ns);
        // x * scales stays in registers between the maximum and the codes
        float f[kTileSlots][8];
        uint32_t amax = 0;
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
#pragma unroll
            for (int q = 0; q < 8; ++q) f[n][q] = xf[n][q];
            mul8(f[n], sm[n][0], sm[n][1]);
            if (MODE == 2) amax = absmax8_products(f[n], amax);
        }
        float dyn = 0.0f;
        if (MODE == 2) {
            amax = wave_max_u32(amax);
            // alternating buffers: a wave can only write this buffer again two picks later,
            // after the next barrier, by which time every wave has read it
            if (lane == 0) red[buf][wave] = amax;
            __syncthreads();
            amax = slots_max(red[buf]);
            dyn = type_max<CT>() / __uint_as_float(amax);
        }
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = lane + (wave * kTileSlots + n) * kWave;
            uint2 packed;
            float gscale = 0.0f;
            if (MODE == 1) {
                packed = static_codes8(f[n]);
            } else if (MODE == 2) {
                packed = dynamic_codes8<CT>(f[n], dyn);
            } else {
                const uint32_t gmax = group_max_u32<kGroup / 8>(absmax8_products(f[n], 0u));
                float gdyn;
                group_dyn<CT>(gmax, gdyn, gscale);
                packed = dynamic_codes8<CT>(f[n], gdyn);
            }
            rsrc_store_stream(orow, 8u * v0 + 512u * n, packed);
            if (MODE == 3)       // the group's first lane; the others aim past the end
                rsrc_store_f32(srow, (v & (kGroup / 8 - 1)) == 0 ? 4u * (v >> 4) : kRsrcPastEnd,
                               gscale);
        }
        if (MODE == 2 && slot0 == 0)                       // wave 0 (uniform): lane 0 stores
            rsrc_store_f32(srow, lane == 0 ? 0u : kRsrcPastEnd, 1.0f / dyn);
    };
    load_pre(0, sa);                                       // n_routed >= 1 here
    for (int j = 0;; j += 2) {
        load_pre(j + 1, sb);
        quant_pick(j, sa, 0);
        if (j + 1 >= n_routed) break;
        load_pre(j + 2, sa);
        quant_pick(j + 1, sb, 1);
        if (j + 2 >= n_routed) break;
    }
}

// ---------------------------------------------------------------------------------------
// per-expert scales: one small workgroup per pick
// ---------------------------------------------------------------------------------------
//
// With an [E][H] scales table each pick is quantized on its own expert's row, so a token's
// K picks share nothing but the token row.  Each pick gets a workgroup of two waves (H up
// to 4096) or four, each holding its share of the row (and the same share of the expert's
// scales row) in registers: the products x * scales, their maximum (mode 2: the waves'
// maxima meet in LDS, one barrier; mode 3: a 128-group is 16 adjacent lanes), the codes and
// the stores, with every load of the pick in flight at once.  A token's K picks thus run side
// by side instead of one after another.  Placement: workgroups are dealt to the eight XCDs in
// turn (workgroup b to XCD b mod 8).  The experts are cut into kPickExpertGroups contiguous
// groups, group g served by XCDs [4g, 4g + 4), so each XCD's L2 holds the scales rows of half
// the experts (3.7 MB at 256 experts and H=7168, instead of a 7.3 MB table that does not fit
// its 4 MB).  Every pick has one candidate workgroup per group, and only the one whose group
// holds the pick's expert goes on: pick k of token t, group g, is workgroup
// 8 (K (t / 4) + k) + 4g + t mod 4, so a token's picks of one group run on one XCD one after
// another, and the token row, read past L2 by the first of them, is an L2 hit for the others
// (these loads keep the default cache policy).  Measured on MI355X at W=8, BS=128, K=8,
// H=7168 (8,192 picks), dispatch with two groups against one (every token's picks on one XCD):
// mode 2 36.0-36.6 against 41.0-41.1 us, mode 1 38.3-38.5 against 41.4 us, per-128-group E4M3
// (mode 3) 42.4-43.2 against 42.2 us and at 12,288 picks 54.6-54.7 against 55.5 us; four and
// eight groups (mode 2) 44.0-44.4 and 55.5-55.8 us (more workgroups that only read an id, each
// token row fetched by more XCDs).

// Used up to kPickKernelMaxPicks picks (larger batches go to the window kernel below, or to
// the token workgroups where a window would hold too few picks per expert).  The crossover
// with the window kernel, measured at H=7168, K=8, 256 experts (dispatch, two expert groups):
// 8,192 picks 36.7-37.0 against 43.7-44.1 us, 10,240 picks 42.1 against 46.3-47.0 us,
// 12,288 picks 46.9-47.0 against 51.0-52.1 us, 16,384 picks 58.6 against 60.7-62.0 us
// (with every token's picks on one XCD the window kernel had been faster from about 9,000
// picks).  Measured on
// MI355X: W=8, BS=128, K=8, H=7168 (8,192 picks) dispatch 41.3 us against 46.7 us with the
// token workgroups (and four waves of four slots per pick against two of seven: 41.3-41.6
// against 41.6-42.0 us, per-128-group E4M3 codes 58.3 against 63.6 us); at W=16, BS=512
// (65,536 picks) 276 us against 265 us for the token workgroups of the time (224 us since
// their pick loop was rebuilt): there each pick's workgroup reads the token row and its
// scales row with little else to overlap, while a token workgroup streams its K picks behind
// a single read of the row.
constexpr long long kPickKernelMaxPicks = 16384;
constexpr int kPickExpertGroups = 2;                 // divides 8
constexpr int kPickGroupXcds = 8 / kPickExpertGroups;

// WAVES waves of SLOTS 64-vector slots each per pick (WAVES * SLOTS * 64 * 8 >= H)
template <int MODE, int CT, int WAVES, int SLOTS>
__global__ __launch_bounds__(kWave * WAVES) void scatter_pick_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const int32_t* __restrict__ seg,
    const float* __restrict__ scales, const float* __restrict__ weights,
    void* __restrict__ expand_x, void* __restrict__ dyn_scales, int32_t* __restrict__ assist,
    float* __restrict__ expand_scales, int W, int E, int BS, int H, int K, int ns,
    long long cap, long long T, int tok_f16)
{
    __shared__ uint32_t red[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int xcd = blockIdx.x & 7;
    const int g = xcd / kPickGroupXcds;                    // expert group this workgroup serves
    const long long jb = (long long)blockIdx.x >> 3;
    const int k = (int)(jb % K);
    const long long tok = (jb / K) * kPickGroupXcds + xcd % kPickGroupXcds;
    if (tok >= T) return;                                  // whole workgroup
    const long long p = tok * K + k;
    const int32_t e = ids[p];
    const int32_t ord = expand_idx[p];
    if (ord < 0 || e < 0 || e >= E) return;                // not routed: whole workgroup
    if ((int)((long long)e * kPickExpertGroups / E) != g) return;   // another group's pick
    const int s = (int)(tok / BS);
    const long long row = (long long)seg[(long long)e * W + s] + ord;
    if (row >= cap) return;

    // this wave's vectors: [base, end) with base a multiple of 64 vectors, so a lane's
    // vectors are base + lane + 64 n and every 128-group is 16 adjacent lanes
    const int NV = H >> 3;
    const int share = ((NV + WAVES - 1) / WAVES + kWave - 1) / kWave * kWave;
    const int base = wave * share;
    const int end = base + share < NV ? base + share : NV;
    const uint4* xr = reinterpret_cast<const uint4*>(x) + tok * NV;
    const float4* sm = reinterpret_cast<const float4*>(scales + (long long)e * H);
    uint4 raw[SLOTS];
    float4 sa[SLOTS], sb[SLOTS];
#pragma unroll
    for (int n = 0; n < SLOTS; ++n) {
        const int v = base + lane + n * kWave;
        if (v < end) {
            raw[n] = xr[v];
            sa[n] = sm[2 * v];
            sb[n] = sm[2 * v + 1];
        }
    }
    if (threadIdx.x == 0) {
        const int i = (int)(tok - (long long)s * BS);
        assist[row * 3 + 0] = s;
        assist[row * 3 + 1] = i;
        assist[row * 3 + 2] = k;
        if (expand_scales) expand_scales[row] = weights[p];
    }
    float f[SLOTS][8];
    uint32_t amax = 0;
#pragma unroll
    for (int n = 0; n < SLOTS; ++n) {
        const int v = base + lane + n * kWave;
        if (v < end) {
            unpack8(raw[n], f[n], tok_f16 != 0);
            mul8(f[n], sa[n], sb[n]);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) f[n][q] = 0.0f;
        }
        if (MODE == 2) amax = absmax8_products(f[n], amax);
    }
    float dyn = 0.0f;
    if (MODE == 2) {
        amax = wave_max_u32(amax);
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        amax = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) amax = amax > red[w] ? amax : red[w];
        dyn = type_max<CT>() / __uint_as_float(amax);
        if (threadIdx.x == 0) static_cast<float*>(dyn_scales)[row] = 1.0f / dyn;
    }
    uint2* out = reinterpret_cast<uint2*>(expand_x) + row * NV;
    float* fscales = static_cast<float*>(dyn_scales);
#pragma unroll
    for (int n = 0; n < SLOTS; ++n) {
        const int v = base + lane + n * kWave;
        uint2 packed;
        float gscale = 0.0f;
        if (MODE == 1) {
            packed = static_codes8(f[n]);
        } else if (MODE == 2) {
            packed = dynamic_codes8<CT>(f[n], dyn);
        } else {
            const uint32_t gmax = group_max_u32<kGroup / 8>(absmax8_products(f[n], 0u));
            float gdyn;
            group_dyn<CT>(gmax, gdyn, gscale);
            packed = dynamic_codes8<CT>(f[n], gdyn);
        }
        if (v >= end) continue;
        store_stream(out + v, packed);
        if (MODE == 3 && (v & (kGroup / 8 - 1)) == 0) fscales[row * ns + (v >> 4)] = gscale;
    }
}

// ---------------------------------------------------------------------------------------
// per-expert scales, larger batches: one workgroup per (token window, expert)
// ---------------------------------------------------------------------------------------
//
// A token workgroup reads the scales rows of its K experts (4H bytes each, twice its token
// row) for every pick; with 256 experts at H=7168 the 7.3 MB table does not fit an XCD's 4 MB
// L2, so about half of those reads go out to the Infinity Cache.  Here the roles are swapped:
// a workgroup holds one expert's scales row in registers and quantizes that expert's picks
// among a window of `win` consecutive tokens (source ranks in turn), reading their token rows.
// The E workgroups of a window run on one XCD (workgroup b runs on XCD b mod 8: window w goes
// to XCD w mod 8, and its E workgroups follow one another there), so a window's token rows
// come from HBM for the first workgroup that needs them and can be L2 hits for the others
// (their loads keep the default cache policy), while each scales row is read once per window.
// Measured at W=16, BS=512, E=256, H=7168, K=8 with 512-token windows: 640 MB read past L2
// per launch instead of 1.03 GB -- 117 MB of scales and each token row about 4.5 times for
// its 8 picks (a window's 7.3 MB of rows do not all stay in L2).  The window's picks of one
// expert fill a run of consecutive packed rows per source rank (segment (e, s) is in token
// order).
// The workgroup finds its picks by scanning the window's ids and expand_idx (L2 hits after
// the first workgroup of the window), listed in (token, pick) order; a pick's row is its
// segment base plus its expand_idx, and the thread that finds it writes its source triple
// and weight.  Then the picks run one after another -- products, their maximum (mode 2: the
// waves' maxima meet in LDS, one barrier per pick), codes, stores -- with the next pick's
// token row in flight meanwhile in the other of two register buffers.
constexpr int kWinMaxTokens = 512;
constexpr int kWinMaxList = 4096;      // win * K: 32 KiB of LDS lists
constexpr int kScanBatch = 4;          // pick loads in flight per lane in the window scan

__device__ __forceinline__ uint4 rsrc_load_u4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int MODE, int CT>
__global__ __launch_bounds__(kWave * kMaxTileWaves) void scatter_window_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const int32_t* __restrict__ seg,
    const float* __restrict__ scales, const float* __restrict__ weights,
    void* __restrict__ expand_x, void* __restrict__ dyn_scales, int32_t* __restrict__ assist,
    float* __restrict__ expand_scales, int W, int E, int BS, int H, int K, int ns,
    long long cap, int win, int tok_f16)
{
    // the expert's picks in the window (at most win * K: a token may list an expert K times):
    // token within the window, and packed row
    extern __shared__ int32_t win_lists[];
    int32_t* list_tok = win_lists;
    int32_t* list_row = win_lists + win * K;
    int32_t* seg_lds = win_lists + 2 * win * K;          // segment bases (e, s) of the window
    __shared__ int32_t wave_cnt[kMaxTileWaves];
    __shared__ uint32_t red[2][kMaxTileWaves];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    // workgroup b = 8 (w / 8 * E + e) + w % 8 serves window w (tokens [w win, w win + win)
    // of the flat (rank, token) order), expert e
    const int xcd = blockIdx.x & 7;
    const long long jb = blockIdx.x >> 3;
    const int e = (int)(jb % E);
    const long long w = (jb / E) * 8 + xcd;
    const long long T = (long long)W * BS;
    const long long tok0 = w * win;
    if (tok0 >= T) return;                                 // whole workgroup
    const int ntok = T - tok0 < win ? (int)(T - tok0) : win;
    const long long p0 = tok0 * K;
    clear_spare_slots(red, nw);
    const int np = ntok * K;
    const int NV = H >> 3;
    float* fscales = static_cast<float*>(dyn_scales);
    uint2* out = reinterpret_cast<uint2*>(expand_x);       // 8 codes per vector

    // the expert's scales slices of this wave's slots, vector v0 + 64 n in slot n (past the
    // row end the range check returns 0)
    const uint32_t slot0 = (uint32_t)__builtin_amdgcn_readfirstlane(wave * kTileSlots * kWave);
    const uint32_t v0 = (uint32_t)lane + slot0;
    float4 sm[kTileSlots][2];
    {
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales + (long long)e * H, 4u * H);
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            sm[n][0] = rsrc_load_f4(sr, 32u * v0 + 2048u * n);
            sm[n][1] = rsrc_load_f4(sr, 32u * v0 + 2048u * n + 16u);
        }
    }

    // list the expert's routed picks in the window in flat (token, pick) order, so the
    // workgroups that run side by side on an XCD walk through the window's token rows
    // together.  Wave w scans the picks [w per_wave, (w + 1) per_wave) twice: first it counts
    // its candidates (ids == e, expand_idx >= 0), then, once every wave's count is in LDS,
    // it writes them behind those of the waves before it.  A row past `cap` is listed as -1
    // (its stores go nowhere).  The segment bases of the ranks the window spans are staged in
    // LDS meanwhile.
    const long long s_lo = tok0 / BS;
    const int span = (int)((tok0 + ntok - 1) / BS - s_lo) + 1;          // <= ntok <= win
    for (int t = threadIdx.x; t < span; t += blockDim.x)
        seg_lds[t] = seg[(long long)e * W + s_lo + t];
    if (threadIdx.x < kMaxTileWaves && (int)threadIdx.x >= nw) wave_cnt[threadIdx.x] = 0;
    const int per_wave = (np + nw * kWave - 1) / (nw * kWave) * kWave;
    const int q_lo = wave * per_wave;
    const int q_hi = q_lo + per_wave < np ? q_lo + per_wave : np;
    auto scan = [&](bool write, int place) -> int {
        for (int q0 = q_lo; q0 < q_hi; q0 += kScanBatch * kWave) {     // uniform per wave
            int32_t pe[kScanBatch], od[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) {                     // all loads in flight
                const int q = q0 + u * kWave + lane;
                pe[u] = -1;
                od[u] = -1;
                if (q < q_hi) {
                    pe[u] = ids[p0 + q];
                    od[u] = expand_idx[p0 + q];
                }
            }
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) {
                const bool hit = pe[u] == e && od[u] >= 0;
                const uint64_t bal = __ballot(hit);
                if (write && hit) {
                    const int q = q0 + u * kWave + lane;
                    const int idx = place + __popcll(bal & ((1ull << lane) - 1ull));
                    const int tl = q / K;
                    const int sr = (int)((tok0 + tl) / BS - s_lo);
                    const long long row = (long long)seg_lds[sr] + od[u];
                    list_tok[idx] = tl;
                    list_row[idx] = row < cap ? (int32_t)row : -1;
                    if (row < cap) {
                        const int s = (int)s_lo + sr;
                        assist[row * 3 + 0] = s;
                        assist[row * 3 + 1] = (int)(tok0 + tl - (long long)s * BS);
                        assist[row * 3 + 2] = q - tl * K;
                        if (expand_scales) expand_scales[row] = weights[p0 + q];
                    }
                }
                place += __popcll(bal);
            }
        }
        return place;
    };
    const int mine = scan(false, 0);
    if (lane == 0) wave_cnt[wave] = mine;
    __syncthreads();
    int place = 0, n_picks = 0;
#pragma unroll
    for (int w2 = 0; w2 < kMaxTileWaves; ++w2) {          // absent waves' counts are 0
        const int c = wave_cnt[w2];
        place += w2 < wave ? c : 0;
        n_picks += c;
    }
    n_picks = __builtin_amdgcn_readfirstlane(n_picks);
    if (n_picks == 0) return;                              // uniform over the workgroup
    scan(true, place);
    __syncthreads();

    // the token row of list entry j, in flight while the previous entry is quantized; past
    // the end of the list the resource is empty and the loads read nothing
    uint4 ra[kTileSlots], rb[kTileSlots];
    auto load_row = [&](int j, uint4 (&dst)[kTileSlots]) {
        const bool in = j < n_picks;                       // uniform
        const int tl = __builtin_amdgcn_readfirstlane(list_tok[in ? j : 0]);
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (tok0 + tl) * H, in ? 2u * H : 0u);
        uint32_t off = 16u * v0;
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) dst[n] = rsrc_load_u4(xr, off + 1024u * n);
    };
    auto quant_pick = [&](int j, const uint4 (&raw)[kTileSlots], int buf) {
        const int prow = __builtin_amdgcn_readfirstlane(list_row[j]);   // -1: past cap
        const long long orow0 = prow < 0 ? 0 : prow;
        const __amdgpu_buffer_rsrc_t orow =
            make_rsrc(out + orow0 * NV, prow < 0 ? 0u : 8u * NV);
        const __amdgpu_buffer_rsrc_t srow =
            make_rsrc(fscales + orow0 * ns, prow < 0 ? 0u : 4u * (uint32_t)ns);
        float f[kTileSlots][8];
        uint32_t amax = 0;
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            unpack8(raw[n], f[n], tok_f16 != 0);
            mul8(f[n], sm[n][0], sm[n][1]);
            if (MODE == 2) amax = absmax8_products(f[n], amax);
        }
        float dyn = 0.0f;
        if (MODE == 2) {
            amax = wave_max_u32(amax);
            // alternating buffers: a wave can only write this buffer again two picks later,
            // after the next barrier, by which time every wave has read it
            if (lane == 0) red[buf][wave] = amax;
            __syncthreads();
            amax = slots_max(red[buf]);
            dyn = type_max<CT>() / __uint_as_float(amax);
        }
#pragma unroll
        for (int n = 0; n < kTileSlots; ++n) {
            const int v = (int)v0 + n * kWave;
            uint2 packed;
            float gscale = 0.0f;
            if (MODE == 1) {
                packed = static_codes8(f[n]);
            } else if (MODE == 2) {
                packed = dynamic_codes8<CT>(f[n], dyn);
            } else {
                const uint32_t gmax = group_max_u32<kGroup / 8>(absmax8_products(f[n], 0u));
                float gdyn;
                group_dyn<CT>(gmax, gdyn, gscale);
                packed = dynamic_codes8<CT>(f[n], gdyn);
            }
            rsrc_store_stream(orow, 8u * v0 + 512u * n, packed);
            if (MODE == 3)       // the group's first lane; the others aim past the end
                rsrc_store_f32(srow, (v & (kGroup / 8 - 1)) == 0 ? 4u * (v >> 4) : kRsrcPastEnd,
                               gscale);
        }
        if (MODE == 2 && slot0 == 0)                       // wave 0 (uniform): lane 0 stores
            rsrc_store_f32(srow, lane == 0 ? 0u : kRsrcPastEnd, 1.0f / dyn);
    };
    load_row(0, ra);
    for (int j = 0;; j += 2) {
        load_row(j + 1, rb);
        quant_pick(j, ra, 0);
        if (j + 1 >= n_picks) break;
        load_row(j + 2, ra);
        quant_pick(j + 1, rb, 1);
        if (j + 2 >= n_picks) break;
    }
}

// Tokens per window for the window kernel, or 0 where it does not pay.  A window is at most
// kWinTokens tokens (and win * K <= kWinMaxList); the batch is cut into a multiple of 8
// windows of equal size, so every XCD gets the same number; and the workgroups must average
// at least kWinMinPicks picks each (win * K >= kWinMinPicks * E), or the scan and the
// scales row of each workgroup are spread over too little work.  Measured on MI355X at
// W=16, BS=512, E=256, H=7168, K=8 (dispatch, int8 per token with per-expert scales):
// windows of 512 tokens 209-223 us, 256 tokens 214-233 us, 128 tokens 226-237 us, against
// 225-237 us for the token workgroups; the scales read past L2 fall from 1.03 GB to 0.63 GB
// per launch.  Up to kPickKernelMaxPicks picks the pick kernel is faster (W=8, BS=128:
// 41 us against 45 us with 128-token windows, before its expert groups; W=16, BS=128:
// 58.6 against 60.7-62.0 us).
constexpr int kWinTokens = 512;
constexpr int kWinMinPicks = 2;
static_assert(kWinTokens <= kWinMaxTokens, "window size");

inline int window_tokens(const Shape& sh)
{
    const long long T = (long long)sh.W * sh.BS;
    const int fit = kWinMaxList / sh.K;
    const int most = kWinTokens < fit ? kWinTokens : fit;
    const long long per_xcd = (T + 8LL * most - 1) / (8LL * most);   // windows per XCD
    const int win = (int)((T + 8 * per_xcd - 1) / (8 * per_xcd));    // <= most
    if ((long long)win * sh.K < (long long)kWinMinPicks * sh.E) return 0;
    return win;
}

// Arguments of every scatter launch.
struct ScatterArgs {
    const void* x;
    const int32_t* ids;
    int32_t* expand_idx;
    const int32_t* seg;
    const float* scales;
    const float* weights;
    void* expand_x;
    void* dyn_scales;
    int32_t* assist;
    float* expand_scales;
    const FusedRoute* fused;    // null: routing comes from the route and scan kernels
};

template <int MODE, int CT, int SK>
hipError_t launch_tile_variant(const Shape& sh, const ScatterArgs& a, hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    if constexpr (SK == kScalesPerExpert) {
        const int win = a.fused ? 0 : window_tokens(sh);
        if (win > 0 && T * sh.K > kPickKernelMaxPicks) {
            const long long windows = (T + win - 1) / win;
            const long long blocks = (windows + 7) / 8 * 8 * sh.E;
            const int slots = ((sh.H >> 3) + kWave - 1) / kWave;
            const int waves = (slots + kTileSlots - 1) / kTileSlots;        // <= kMaxTileWaves
            const size_t lds = sizeof(int32_t) * ((size_t)2 * win * sh.K + win);
            hipLaunchKernelGGL((scatter_window_kernel<MODE, CT>), dim3((unsigned)blocks),
                               dim3(kWave * waves), lds, stream,
                               static_cast<const uint16_t*>(a.x), a.ids, a.expand_idx, a.seg,
                               a.scales, a.weights, a.expand_x, a.dyn_scales, a.assist,
                               a.expand_scales, sh.W, sh.E, sh.BS, sh.H, sh.K,
                               sh.scales_per_row, (long long)sh.cap, win, sh.tok_f16);
            return hipGetLastError();
        }
        if (!a.fused && T * sh.K <= kPickKernelMaxPicks) {
            // one workgroup per (pick, expert group): the matching one quantizes the pick
            const long long blocks =
                (T + kPickGroupXcds - 1) / kPickGroupXcds * 8 * sh.K;
#define MOE_DC_PICK(WV, SL)                                                                    \
    hipLaunchKernelGGL((scatter_pick_kernel<MODE, CT, WV, SL>), dim3((unsigned)blocks),         \
                       dim3(kWave * WV), 0, stream, static_cast<const uint16_t*>(a.x), a.ids,   \
                       a.expand_idx, a.seg, a.scales, a.weights, a.expand_x, a.dyn_scales,     \
                       a.assist, a.expand_scales, sh.W, sh.E, sh.BS, sh.H, sh.K,               \
                       sh.scales_per_row, (long long)sh.cap, T, sh.tok_f16)
            if (sh.H <= 2 * 4 * kWave * 8) MOE_DC_PICK(2, 4);
            else MOE_DC_PICK(4, 4);
#undef MOE_DC_PICK
            return hipGetLastError();
        }
    }
    const int slots = ((sh.H >> 3) + kWave - 1) / kWave;
    int waves = (slots + kTileSlots - 1) / kTileSlots;              // <= kMaxTileWaves
    size_t lds = 0;
    FusedRoute fr{};
    if (a.fused) {
        fr = *a.fused;
        if (waves < kFusedMinWaves) waves = kFusedMinWaves;
        lds = ((size_t)sh.E * sh.W + 1) * sizeof(int32_t);
    }
#define MOE_DC_TILE_LAUNCH(F)                                                                   \
    hipLaunchKernelGGL((scatter_tile_kernel<MODE, CT, SK, F>), dim3((unsigned)(T + (F ? 1 : 0))), \
                       dim3(kWave * waves), lds, stream, static_cast<const uint16_t*>(a.x),     \
                       a.ids, a.expand_idx, a.seg, a.scales, a.weights, a.expand_x,            \
                       a.dyn_scales, a.assist, a.expand_scales, sh.W, sh.E, sh.BS, sh.H, sh.K, \
                       sh.scales_per_row, (long long)sh.cap, sh.scale_format, fr, sh.L,         \
                       sh.mask_kind, sh.etn_type, sh.tok_f16)
    if (a.fused) MOE_DC_TILE_LAUNCH(true);
    else MOE_DC_TILE_LAUNCH(false);
#undef MOE_DC_TILE_LAUNCH
    return hipGetLastError();
}

template <int MODE, int CT>
hipError_t launch_tile_scales(const Shape& sh, const ScatterArgs& a, hipStream_t stream)
{
#define MOE_DC_TILE(SK) launch_tile_variant<MODE, CT, SK>(sh, a, stream)
    switch (sh.scales_kind) {
    case kScalesNone:
        if constexpr (MODE == 1) return hipErrorInvalidValue;    // mode 1 needs scales
        else return MOE_DC_TILE(kScalesNone);
    case kScalesScalar:
        return MOE_DC_TILE(kScalesScalar);
    case kScalesShared:
        return MOE_DC_TILE(kScalesShared);
    case kScalesPerExpert:
        return MOE_DC_TILE(kScalesPerExpert);
    default:
        return hipErrorInvalidValue;
    }
#undef MOE_DC_TILE
}

hipError_t launch_tile(const Shape& sh, const ScatterArgs& a, hipStream_t stream)
{
#define MOE_DC_ARGS sh, a, stream
    const int ct = sh.code_type;
    switch (sh.quant_mode) {
    case 0:
        return launch_tile_variant<0, kCodeBf16, kScalesNone>(MOE_DC_ARGS);
    case 1:
        return launch_tile_scales<1, kCodeInt8>(MOE_DC_ARGS);
    case 2:
        if (ct == kCodeInt8) return launch_tile_scales<2, kCodeInt8>(MOE_DC_ARGS);
        if (ct == kCodeE4m3) return launch_tile_scales<2, kCodeE4m3>(MOE_DC_ARGS);
        return launch_tile_scales<2, kCodeE5m2>(MOE_DC_ARGS);
    case 3:
        if (ct == kCodeE4m3) return launch_tile_scales<3, kCodeE4m3>(MOE_DC_ARGS);
        return launch_tile_scales<3, kCodeE5m2>(MOE_DC_ARGS);
    case 4:
        if (ct == kCodeE4m3) return launch_tile_variant<4, kCodeE4m3, kScalesNone>(MOE_DC_ARGS);
        if (ct == kCodeE2m1) return launch_tile_variant<4, kCodeE2m1, kScalesNone>(MOE_DC_ARGS);
        return launch_tile_variant<4, kCodeE5m2, kScalesNone>(MOE_DC_ARGS);
    case 5:
        if (ct == kCodeE4m3) return launch_tile_variant<5, kCodeE4m3, kScalesNone>(MOE_DC_ARGS);
        if (ct == kCodeE2m1) return launch_tile_variant<5, kCodeE2m1, kScalesNone>(MOE_DC_ARGS);
        return launch_tile_variant<5, kCodeE5m2, kScalesNone>(MOE_DC_ARGS);
    default:
        return hipErrorInvalidValue;
    }
#undef MOE_DC_ARGS
}

// ---------------------------------------------------------------------------------------
// element-wise fallback: one workgroup per token, one element per lane
// ---------------------------------------------------------------------------------------

constexpr int kElemThreads = 1024;
constexpr int kElemPerLane = 8;      // H <= 8192 = 1024 lanes x 8
constexpr int kElemWaves = kElemThreads / kWave;

__device__ __forceinline__ uint32_t fp8_code_rt(int ct, float v)
{
    return ct == kCodeE4m3 ? e4m3_code(v) : ct == kCodeE5m2 ? e5m2_code(v) : e2m1_code(v);
}

__device__ __forceinline__ uint32_t dynamic_code_rt(int ct, float v)
{
    if (ct == kCodeInt8) return int8_code(v);
    return v != v ? 0u : fp8_code_rt(ct, v);
}

__device__ __forceinline__ float type_max_rt(int ct)
{
    return ct == kCodeInt8 ? 127.0f : ct == kCodeE4m3 ? 448.0f : 57344.0f;
}

// The variant (mode, code type, scales kind, E8M0 scales) is a runtime argument here: this
// kernel serves odd sizes and alignments only, where clarity matters more than speed.
// Requires blockDim.x == 1024 for mode 3 (so a 128-element group is two whole waves of one
// pass), which holds for every valid H (>= 1024).
__global__ __launch_bounds__(kElemThreads) void scatter_elem_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ expand_idx, const int32_t* __restrict__ seg,
    const float* __restrict__ scales, const float* __restrict__ weights,
    void* __restrict__ expand_x, void* __restrict__ dyn_scales, int32_t* __restrict__ assist,
    float* __restrict__ expand_scales, int W, int E, int BS, int H, int K, int ns,
    long long cap, int mode, int ct, int sk, int sfmt, int tok_f16)
{
    __shared__ long long row_of[kMaxK];
    __shared__ int32_t exp_of[kMaxK];
    __shared__ uint32_t red[kElemWaves];
    __shared__ uint32_t gred[kElemPerLane][kElemWaves];

    const long long tok = blockIdx.x;
    const int s = (int)(tok / BS);
    const int i = (int)(tok - (long long)s * BS);
    const int t = threadIdx.x;
    const int nt = blockDim.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    float* fscales = static_cast<float*>(dyn_scales);
    uint8_t* bscales = static_cast<uint8_t*>(dyn_scales);

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
            if (expand_scales) expand_scales[row] = weights[tok * K + t];
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

    if (mode == 0) {
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
    const int nb = (H + kMxBlock - 1) / kMxBlock;
    const float tmax = type_max_rt(ct);

    // Per-expert scales make the codes per pick; otherwise one pass serves all K picks.
    const int passes = sk == kScalesPerExpert ? K : 1;
    for (int pk = 0; pk < passes; ++pk) {
        if (sk == kScalesPerExpert && row_of[pk] < 0) continue;   // uniform over the block
        const float* pre = sk == kScalesPerExpert ? scales + (long long)exp_of[pk] * H : scales;
        float f[kElemPerLane];
        uint32_t a[kElemPerLane];
        uint32_t amax = 0;
#pragma unroll
        for (int n = 0; n < kElemPerLane; ++n) {
            const int h = t + n * nt;
            f[n] = 0.0f;
            if (h < H) {
                f[n] = tok_lo_rt(raw[n], tok_f16 != 0);
                if (sk == kScalesScalar) f[n] = f[n] * pre[0];
                if (sk == kScalesShared || sk == kScalesPerExpert) f[n] = f[n] * pre[h];
            }
            a[n] = __float_as_uint(f[n]) & 0x7FFFFFFFu;
            amax = amax > a[n] ? amax : a[n];
        }
        float dyn_tok = 0.0f;
        if (mode == 2) {
            amax = block_max_u32(amax, red);
            dyn_tok = tmax / __uint_as_float(amax);
        }
        if (mode == 3) {
            // each 128-element group is the two waves 2j, 2j+1 of one pass
#pragma unroll
            for (int n = 0; n < kElemPerLane; ++n) {
                const uint32_t w = wave_max_u32(a[n]);
                if (lane == 0) gred[n][wave] = w;
            }
            __syncthreads();
        }
#pragma unroll
        for (int n = 0; n < kElemPerLane; ++n) {
            const int h = t + n * nt;
            if (n * nt >= H) break;                        // uniform across the workgroup
            uint32_t code = 0;
            float scale = 0.0f;
            uint32_t sbyte = 0;
            bool lead = false;
            int sidx = 0;
            if (mode == 1) {
                code = int8_code(f[n]);
            } else if (mode == 2) {
                code = dynamic_code_rt(ct, f[n] * dyn_tok);
            } else if (mode == 3) {
                const int w0 = wave & ~1;
                const uint32_t g = gred[n][w0] > gred[n][w0 + 1] ? gred[n][w0] : gred[n][w0 + 1];
                const float dyn = tmax / __uint_as_float(g);
                code = dynamic_code_rt(ct, f[n] * dyn);
                scale = 1.0f / dyn;
                lead = (h % kGroup) == 0;
                sidx = h / kGroup;
            } else {
                const uint32_t bm = group_max_u32<kMxBlock>(a[n]);
                const int se = mode == 4
                    ? (ct == kCodeE4m3   ? mx_shared_exp<4, kCodeE4m3>(bm)
                       : ct == kCodeE5m2 ? mx_shared_exp<4, kCodeE5m2>(bm)
                                         : mx_shared_exp<4, kCodeE2m1>(bm))
                    : (ct == kCodeE4m3   ? mx_shared_exp<5, kCodeE4m3>(bm)
                       : ct == kCodeE5m2 ? mx_shared_exp<5, kCodeE5m2>(bm)
                                         : mx_shared_exp<5, kCodeE2m1>(bm));
                const float inv = __uint_as_float((uint32_t)(127 - se) << 23);   // 2^-se
                code = fp8_code_rt(ct, f[n] * inv);
                scale = sfmt == 2 ? inv : pow2f(se);
                sbyte = (uint32_t)(se + 127);
                lead = (h % kMxBlock) == 0;
                sidx = h / kMxBlock;
            }
            // E2M1: the even element of each pair writes both codes as one byte (H is even)
            const uint32_t next = __shfl_down(code, 1, kWave);
            if (h >= H) continue;
            const bool fp4 = ct == kCodeE2m1;
            for (int k = 0; k < K; ++k) {
                const long long row = sk == kScalesPerExpert ? (k == pk ? row_of[pk] : -1)
                                                             : row_of[k];
                if (row < 0) continue;
                if (!fp4) out[row * H + h] = (uint8_t)code;
                else if ((h & 1) == 0) out[row * (H / 2) + h / 2] = (uint8_t)(code | (next << 4));
                if (lead) {
                    if (sfmt == 1) bscales[row * ns + sidx] = (uint8_t)sbyte;
                    else fscales[row * ns + sidx] = scale;
                }
            }
        }
        if (t == 0) {
            for (int k = 0; k < K; ++k) {
                const long long row = sk == kScalesPerExpert ? (k == pk ? row_of[pk] : -1)
                                                             : row_of[k];
                if (row < 0) continue;
                if (mode == 2) fscales[row] = 1.0f / dyn_tok;
                if (mode >= 4 && ns > nb) {
                    if (sfmt == 1) bscales[row * ns + nb] = 0;
                    else fscales[row * ns + nb] = 0.0f;
                }
            }
        }
        if (mode == 3) __syncthreads();                    // gred is reused by the next pick
    }
}

hipError_t launch_elem(const Shape& sh, const ScatterArgs& a, hipStream_t stream)
{
    const long long T = (long long)sh.W * sh.BS;
    const int want = (sh.H + kWave - 1) / kWave * kWave;
    const int threads = want < kElemThreads ? want : kElemThreads;
    if (sh.quant_mode == 3 && threads != kElemThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_elem_kernel, dim3((unsigned)T), dim3(threads), 0, stream,
                       static_cast<const uint16_t*>(a.x), a.ids, a.expand_idx, a.seg, a.scales,
                       a.weights, a.expand_x, a.dyn_scales, a.assist, a.expand_scales, sh.W,
                       sh.E, sh.BS, sh.H, sh.K, sh.scales_per_row, (long long)sh.cap,
                       sh.quant_mode, sh.code_type, sh.scales_kind, sh.scale_format, sh.tok_f16);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scatter(const Shape& sh, const void* x, const int32_t* expert_ids,
                          int32_t* expand_idx, const int32_t* seg, const float* scales,
                          const float* expert_scales, void* expand_x, void* dynamic_scales,
                          int32_t* assist_info, float* expand_scales, bool vectorized,
                          const FusedRoute* fused, hipStream_t stream)
{
    if (fused && (!vectorized || !fused_route_fits(sh))) return hipErrorInvalidValue;
    const ScatterArgs a{x,        expert_ids,     expand_idx,  seg,          scales,
                        expert_scales, expand_x, dynamic_scales, assist_info, expand_scales,
                        fused};
    return vectorized ? launch_tile(sh, a, stream) : launch_elem(sh, a, stream);
}

}  // namespace moe_dc
