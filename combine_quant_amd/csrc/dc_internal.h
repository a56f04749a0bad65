// dc_internal.h -- launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_dc.h"

namespace moe_dc {

// Records `msg` as the calling thread's moe_dc_last_error() text and returns `st`.
moe_status set_error(moe_status st, const char* msg);

struct Shape;

// Every host-side rule of moe_dispatch except those on the workspace: the config, the
// required pointers and the pairings of optional ones.  Fills *out (if not null) on success.
moe_status check_dispatch_args(const moe_dc_config* cfg, const void* x,
                               const int32_t* expert_ids, const float* scales,
                               const uint8_t* x_active_mask, const float* expert_scales,
                               const void* expand_x, const void* dynamic_scales,
                               const int32_t* expand_idx, const int32_t* assist_info,
                               const int32_t* ep_recv_count, const int64_t* expert_token_nums,
                               const int64_t* recv_offsets, const float* expand_scales,
                               Shape* out);

// Element types of expand_x (the values of moe_dtype in the C ABI).
enum CodeType : int32_t {
    kCodeBf16 = 0, kCodeInt8 = 1, kCodeE4m3 = 2, kCodeE5m2 = 3, kCodeE2m1 = 4
};

// Shapes of the quantization scales tensor (the values of moe_scales_kind).
enum ScalesKind : int32_t {
    kScalesNone = 0, kScalesScalar = 1, kScalesShared = 2, kScalesPerExpert = 3
};

// Validated shape of one dispatch/combine problem (see moe_dc_config in include/moe_dc.h).
struct Shape {
    int32_t W, E, L, BS, H, K;
    int32_t quant_mode;
    int32_t code_type;       // CodeType of expand_x
    int32_t scales_kind;     // ScalesKind of the scales tensor
    int32_t scale_format;    // MX scales: 0 fp32 2^se, 1 E8M0 bytes, 2 fp32 2^-se
    int32_t zero_end;        // E + zero_expert_num
    int32_t id_end;          // E + zero_expert_num + copy_expert_num
    int32_t etn_type;
    int32_t mask_kind;
    int32_t scales_per_row;  // 0, 1, Ceil(H,128) or Align2(Ceil(H,32))
    int32_t tok_f16;         // 1: token elements are IEEE binary16, 0: bf16
    int64_t cap;
};

// Workspace layout of moe_dispatch, each part 256-byte aligned:
//   [0, 256)      the checked-ids word (int32 at 0; written only with MOE_DC_FLAG_CHECK_IDS)
//   seg           one int32 per (expert e, source rank s) at e*W + s: the route kernel stores
//                 the pick counts there, the scan kernel overwrites each with the exclusive
//                 running total, i.e. the first packed row of that (expert, source) segment
//   bad counts    one int32 per source rank: its active picks with an id outside [0, E+Z+C)
//   group totals  only when E*W > kScanMaxFlat: one int32 per group of ranks of the
//                 two-launch scan (at most W groups)
inline size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
constexpr size_t kWsSegOffset = 256;
constexpr long long kScanMaxFlat = 16384;   // E*W the one-workgroup scan takes in one pass
inline size_t ws_bad_counts_offset(const Shape& s)
{
    return kWsSegOffset + round256((size_t)s.E * (size_t)s.W * sizeof(int32_t));
}
inline size_t ws_scan_totals_offset(const Shape& s)
{
    return ws_bad_counts_offset(s) + round256((size_t)s.W * sizeof(int32_t));
}
inline size_t workspace_bytes(const Shape& s)
{
    const bool grouped = (long long)s.E * s.W > kScanMaxFlat;
    return ws_scan_totals_offset(s) + (grouped ? round256((size_t)s.W * sizeof(int32_t)) : 0);
}

// Routing: counts per (expert, source) and the final expand_idx.  With bad_counts (else
// null), each source rank's count of active picks whose id lies outside [0, id_end).
hipError_t launch_route(const Shape& s, const int32_t* expert_ids, const uint8_t* mask,
                        int32_t* expand_idx, int32_t* seg, int32_t* bad_counts,
                        hipStream_t stream);

// Receive-side prefix sums: seg counts -> segment bases (in place) + the three outputs.
// With bad_word (else null), the sum of the W bad_counts.  totals: the workspace's group
// totals (used only when E*W > kScanMaxFlat).
hipError_t launch_scan(const Shape& s, int32_t* seg, int32_t* ep_recv_count,
                       int64_t* expert_token_nums, int64_t* recv_offsets,
                       const int32_t* bad_counts, int32_t* bad_word, int32_t* totals,
                       hipStream_t stream);

// Small batches route inside the scatter launch: every workgroup recomputes the counts and
// their prefix sums in LDS (W*BS*K ids, E*W counters) instead of reading them from the route
// and scan kernels.  The outputs those kernels would write are written by the scatter launch.
struct FusedRoute {
    const uint8_t* mask;
    int32_t* ep_recv_count;
    int64_t* expert_token_nums;
    int64_t* recv_offsets;
    int32_t* bad_word;      // null, or the checked-ids word
    int32_t id_end;         // E + zero + copy experts
};
constexpr long long kFusedMaxPicks = 2048;   // W*BS*K (measured crossover: 2048-4096)
constexpr long long kFusedMaxCounts = 4096;  // E*W (LDS words)

inline bool fused_route_fits(const Shape& s)
{
    return (long long)s.W * s.BS * s.K <= kFusedMaxPicks &&
           (long long)s.E * s.W <= kFusedMaxCounts;
}

// Quantize and scatter every routed pick to its packed row, with scales and source triple.
// expand_scales (nullable) receives each row's pick weight from expert_scales.  With
// `fused` (vectorized launches only) the launch also does the routing: expand_idx is then an
// output and seg is not used.
hipError_t launch_scatter(const Shape& s, const void* x, const int32_t* expert_ids,
                          int32_t* expand_idx, const int32_t* seg, const float* scales,
                          const float* expert_scales, void* expand_x, void* dynamic_scales,
                          int32_t* assist_info, float* expand_scales, bool vectorized,
                          const FusedRoute* fused, hipStream_t stream);

// Weighted top-K gather.
hipError_t launch_combine(const Shape& s, const void* expert_out, const int32_t* expert_ids,
                          const int32_t* expand_idx, const float* expert_scales,
                          const int32_t* ep_recv_count, const int64_t* recv_offsets,
                          const uint8_t* mask, const void* ori_x, void* y, bool vectorized,
                          hipStream_t stream);

// Weighted top-K gather over int8 block-quantized expert rows (codes [cap][H], fp32 scales
// [cap][Ceil(H,8)]).
hipError_t launch_combine_int8(const Shape& s, const int8_t* codes, const float* qscales,
                               const int32_t* expert_ids, const int32_t* expand_idx,
                               const float* expert_scales, const int32_t* ep_recv_count,
                               const int64_t* recv_offsets, const uint8_t* mask,
                               const void* ori_x, void* y, bool vectorized, hipStream_t stream);

// Scatter-back combine: rows sent back to slots by their assist_info triples, then the
// per-token K-sum (+ the shared expert's output when shared_x is not null).  slot_rows is
// scratch of W*BS*K int32.
hipError_t launch_combine_scatter(const Shape& s, const void* expert_out,
                                  const int32_t* assist_info, const int64_t* recv_offsets,
                                  const int32_t* expert_ids, const float* expert_scales,
                                  const uint8_t* mask, const void* ori_x, const void* shared_x,
                                  void* y, int32_t* slot_rows, bool vectorized,
                                  hipStream_t stream);

inline size_t combine_scatter_workspace_bytes(const Shape& s)
{
    size_t b = (size_t)s.W * (size_t)s.BS * (size_t)s.K * sizeof(int32_t);
    return (b + 255) & ~(size_t)255;
}

// Expert-side int8 block quantization of the rows [0, recv_offsets[W]).
hipError_t launch_combine_quantize(const Shape& s, const void* expert_out,
                                   const int64_t* recv_offsets, int8_t* codes, float* qscales,
                                   bool vectorized, hipStream_t stream);

}  // namespace moe_dc
