// noalloc.hip -- moe_dispatch for callers that cannot allocate device memory.
//
// moe_dispatch_no_workspace runs exactly moe_dispatch (same kernels, same outputs) with its
// workspace taken from `scratch`, a file-scope device array of kNoAllocScratchBytes that
// every GPU the library runs on holds from the module's load until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and only
// that address is ever passed to a kernel.
//
// The dispatch workspace needs no initialisation (the route kernel writes every count before
// the scan reads it), so nothing is cleared between calls; calls that overlap on one GPU
// share the array and race.
#include "moe_dc.h"
#include "dc_internal.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)1 << 20;   // 1 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null: not yet)

// Device address of this device's copy of `scratch`, looked up on the first call.
hipError_t scratch_address(int device, void** out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_dispatch_no_workspace(
    const moe_dc_config* cfg, const void* x, const int32_t* expert_ids, const float* scales,
    const uint8_t* x_active_mask, const float* expert_scales, void* expand_x,
    void* dynamic_scales, int32_t* expand_idx, int32_t* assist_info, int32_t* ep_recv_count,
    int64_t* expert_token_nums, int64_t* recv_offsets, float* expand_scales, void* stream)
{
    // every host-side rule first: nothing below touches the device for a rejected call
    const moe_status st = moe_dc::check_dispatch_args(
        cfg, x, expert_ids, scales, x_active_mask, expert_scales, expand_x, dynamic_scales,
        expand_idx, assist_info, ep_recv_count, expert_token_nums, recv_offsets, expand_scales,
        nullptr);
    if (st != MOE_OK) return st;
    if (cfg->flags & MOE_DC_FLAG_CHECK_IDS)
        return moe_dc::set_error(MOE_ERR_INVALID_ARG,
                                "MOE_DC_FLAG_CHECK_IDS leaves its count in the caller's "
                                "workspace; use moe_dispatch for it");
    const size_t need = moe_dc_dispatch_workspace_bytes(cfg);
    if (need > kNoAllocScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof msg,
                 "this config needs %zu bytes of dispatch workspace; the static scratch "
                 "holds %zu (use moe_dispatch with a workspace)",
                 need, kNoAllocScratchBytes);
        return moe_dc::set_error(MOE_ERR_WORKSPACE, msg);
    }
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= kMaxDevices)) e = hipErrorInvalidDevice;
    void* ws = nullptr;
    if (e == hipSuccess) e = scratch_address(device, &ws);
    if (e != hipSuccess)
        return moe_dc::set_error(MOE_ERR_DEVICE, hipGetErrorString(e));
    return moe_dispatch(cfg, x, expert_ids, scales, x_active_mask, expert_scales, expand_x,
                        dynamic_scales, expand_idx, assist_info, ep_recv_count,
                        expert_token_nums, recv_offsets, expand_scales, ws,
                        kNoAllocScratchBytes, stream);
}
