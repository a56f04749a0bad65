// selfcheck.hip -- exhaustive GPU checks of the instruction-level conversions the dispatch
// kernels use (dc_convert.h) against the bit-level encoders and the correctly rounded division
// they stand in for.  Not part of the dispatch/combine library (libmoe_dc.so); built as
// libmoe_dc_selfcheck.so for the tests.
//
//   codes: every binary32 bit pattern that is not a NaN (infinities included), eight
//          consecutive patterns per call of fp8_codes8_hw<E4M3>, fp8_codes8_hw<E5M2> and
//          fp4_word_hw, each code compared with e4m3_code, e5m2_code and e2m1_code; and every
//          bit pattern (NaNs included) through static_int8_codes8 against int8_code
//   division: every binary32 b with the sign bit clear (zero, subnormals, infinity and NaNs
//          included), div_rn<8>(448, b), div_rn<15>(57344, b) and div_rn<1>(1, b) compared bit
//          for bit with the correctly rounded quotient
#include "dc_convert.h"

#include <hip/hip_runtime.h>

namespace {

using namespace moe_dc;

constexpr int kPer = 256;                 // bit patterns per thread
constexpr int kThreads = 256;
constexpr int kCounts = 7;

// mismatch counters: 0 E4M3, 1 E5M2, 2 E2M1, 3 448 / b, 4 57344 / b, 5 1 / b, 6 int8
__global__ __launch_bounds__(kThreads) void check_codes_kernel(unsigned long long* bad)
{
    const unsigned long long t = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x;
    const unsigned long long first = t * kPer;            // the grid covers 2^32 patterns
    unsigned long long n4 = 0, n5 = 0, n2 = 0, n8 = 0;
    for (int j = 0; j < kPer; j += 8) {
        float all[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) all[q] = __uint_as_float((uint32_t)(first + j + q));
        const uint2 c8 = static_int8_codes8(all);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t w8 = q < 4 ? c8.x : c8.y;
            n8 += ((w8 >> (8 * (q & 3))) & 0xFFu) != (int8_code(all[q]) & 0xFFu);
        }
        float v[8];
        bool cmp[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t u = (uint32_t)(first + j + q);
            const bool nan = (u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu) != 0u;
            v[q] = nan ? 0.0f : __uint_as_float(u);
            cmp[q] = !nan;
        }
        const uint2 c4 = fp8_codes8_hw<kCodeE4m3>(v);
        const uint2 c5 = fp8_codes8_hw<kCodeE5m2>(v);
        const uint32_t c2 = fp4_word_hw(v);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (!cmp[q]) continue;
            const uint32_t w4 = q < 4 ? c4.x : c4.y, w5 = q < 4 ? c5.x : c5.y;
            n4 += ((w4 >> (8 * (q & 3))) & 0xFFu) != e4m3_code(v[q]);
            n5 += ((w5 >> (8 * (q & 3))) & 0xFFu) != e5m2_code(v[q]);
            n2 += ((c2 >> (4 * q)) & 0xFu) != e2m1_code(v[q]);
        }
    }
    if (n4) atomicAdd(&bad[0], n4);
    if (n5) atomicAdd(&bad[1], n5);
    if (n2) atomicAdd(&bad[2], n2);
    if (n8) atomicAdd(&bad[6], n8);
}

__global__ __launch_bounds__(kThreads) void check_division_kernel(unsigned long long* bad)
{
    const unsigned long long t = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x;
    const unsigned long long first = t * kPer;            // the grid covers 2^31 patterns
    unsigned long long n[3] = {0, 0, 0};
    for (int j = 0; j < kPer; ++j) {
        const float b = __uint_as_float((uint32_t)(first + j));
        n[0] += __float_as_uint(div_rn<8>(448.0f, b)) != __float_as_uint(448.0f / b);
        n[1] += __float_as_uint(div_rn<15>(57344.0f, b)) != __float_as_uint(57344.0f / b);
        n[2] += __float_as_uint(div_rn<1>(1.0f, b)) != __float_as_uint(1.0f / b);
    }
#pragma unroll
    for (int m = 0; m < 3; ++m)
        if (n[m]) atomicAdd(&bad[3 + m], n[m]);
}

}  // namespace

extern "C" {

// Runs both checks on the current device and copies the seven mismatch counts (E4M3, E5M2,
// E2M1 codes; 448 / b, 57344 / b, 1 / b; static int8 codes) to the host array `counts`.
// Allocates 56 bytes of device memory for the counters and frees them; synchronizes the
// device.  Returns a hipError_t value (0 on success).
int moe_dc_selfcheck_conversions(unsigned long long* counts)
{
    if (!counts) return (int)hipErrorInvalidValue;
    unsigned long long* bad = nullptr;
    hipError_t e = hipMalloc(&bad, kCounts * sizeof(unsigned long long));
    if (e != hipSuccess) return (int)e;
    e = hipMemset(bad, 0, kCounts * sizeof(unsigned long long));
    if (e == hipSuccess) {
        hipLaunchKernelGGL(check_codes_kernel, dim3((unsigned)((1ull << 32) / kPer / kThreads)),
                           dim3(kThreads), 0, 0, bad);
        hipLaunchKernelGGL(check_division_kernel,
                           dim3((unsigned)((1ull << 31) / kPer / kThreads)), dim3(kThreads), 0,
                           0, bad);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess)
        e = hipMemcpy(counts, bad, kCounts * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    const hipError_t f = hipFree(bad);
    return (int)(e != hipSuccess ? e : f);
}

}  // extern "C"
