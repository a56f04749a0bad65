// ceiling.hip -- measurement kernels for bench.py: the access patterns of the dispatch scatter
// and of the combine gather with the arithmetic taken out, so their rates bound what the real
// kernels can reach on this chip.  Not part of the dispatch/combine library (libmoe_dc.so);
// built as libmoe_dc_ceiling.so.
//
//   ceiling_scatter_copy  one workgroup per token: the token's bf16 row is read once (16-byte
//                         non-temporal loads) and its H high bytes are stored to each of the
//                         token's K destination rows (8-byte non-temporal stores) -- the
//                         scatter's reads and writes, in its order, without the quantization
//   ceiling_write_rows    one wave per destination row, rows visited in a given order (for
//                         instance the scatter's token-major order) or in sequence: the
//                         scatter's writes alone
//   ceiling_gather_sum    one wave task per (token, 128 16-byte vectors): the K source rows of
//                         the token's picks are read (16-byte non-temporal loads, all in
//                         flight) and combined with one integer add per element word, then
//                         the result stored -- the combine's reads and writes without its
//                         fp32 arithmetic
//   ceiling_write_chunks  the same number of bytes written in address order by one-shot
//                         workgroups that each store one chunk (one 16-byte store per lane):
//                         with 4 KiB chunks (four waves) the fastest write shape measured on
//                         this chip, for scale; other chunk sizes show how much that shape
//                         matters
//   ceiling_read_chunks   the gather's read bytes read in address order by one-shot workgroups,
//                         one chunk each (one 16-byte non-temporal load per lane): the chip's
//                         sequential read rate, for scale
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_nt(uint2* p, uint2 o)
{
    const u32x2_t v = {o.x, o.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

__device__ __forceinline__ void store_nt(uint4* p, uint4 o)
{
    const u32x4_t v = {o.x, o.y, o.z, o.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

constexpr int kWave = 64;
constexpr int kMaxK = 16;

// blockDim = H / 16 threads (H a multiple of 1024, at most 8192): thread t owns vectors
// (t % 64) + 64 * (2 * (t / 64) + n), n = 0, 1, of 8 bf16 elements each
__global__ __launch_bounds__(512) void ceiling_scatter_copy_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ rows, uint8_t* __restrict__ out,
    int H, int K)
{
    __shared__ int32_t dest[kMaxK];
    const long long tok = blockIdx.x;
    const int t = threadIdx.x;
    const int NV = H / 8;
    if (t < K) dest[t] = rows[tok * K + t];
    const uint4* xr = reinterpret_cast<const uint4*>(x + tok * H);
    uint4 a[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int v = (t & (kWave - 1)) + ((t / kWave) * 2 + n) * kWave;
        if (v < NV) a[n] = load_nt(xr + v);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int v = (t & (kWave - 1)) + ((t / kWave) * 2 + n) * kWave;
        if (v >= NV) continue;
        const uint2 c = make_uint2(__builtin_amdgcn_perm(a[n].y, a[n].x, 0x07050301u),
                                   __builtin_amdgcn_perm(a[n].w, a[n].z, 0x07050301u));
        for (int k = 0; k < K; ++k)
            if (dest[k] >= 0) store_nt(reinterpret_cast<uint2*>(out + (long long)dest[k] * H) + v, c);
    }
}

__global__ __launch_bounds__(256) void ceiling_write_rows_kernel(
    uint8_t* __restrict__ out, const int32_t* __restrict__ order, long long rows, int H)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const long long t = (long long)blockIdx.x * 4 + wave;
    if (t >= rows) return;
    const long long row = order ? order[t] : t;
    uint2* o = reinterpret_cast<uint2*>(out + row * H);
    for (int v = lane; v < H / 8; v += kWave) store_nt(o + v, make_uint2((uint32_t)row, (uint32_t)v));
}

// one wave task = one token x two 64-vector slots; src[tok * K + k] is the row of pick k
// (or -1); rows and y are bf16 [.][H]
template <int KMAX>
__global__ __launch_bounds__(256) void ceiling_gather_sum_kernel(
    const uint4* __restrict__ rows, const int32_t* __restrict__ src, uint4* __restrict__ y,
    long long T, int H, int K, int tasks_per_token)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const long long task = (long long)blockIdx.x * 4 + wave;
    const long long tok = task / tasks_per_token;
    if (tok >= T) return;
    const int slot0 = (int)(task - tok * tasks_per_token) * 2;
    const int NV = H / 8;
    const int mine = lane < K ? src[tok * K + lane] : -1;
    int r[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) r[k] = __builtin_amdgcn_readlane(mine, k);
    uint4 buf[2][KMAX];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v >= NV) continue;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K && r[k] >= 0) buf[n][k] = load_nt(rows + (long long)r[k] * NV + v);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int v = lane + (slot0 + n) * kWave;
        if (v >= NV) continue;
        uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K || r[k] < 0) continue;
            acc.x += buf[n][k].x; acc.y += buf[n][k].y; acc.z += buf[n][k].z; acc.w += buf[n][k].w;
        }
        store_nt(y + tok * NV + v, acc);
    }
}

// workgroup b (blockDim lanes) writes the 16-byte units [b * blockDim, (b + 1) * blockDim) of
// out, n16 units in all
__global__ __launch_bounds__(1024) void ceiling_write_chunks_kernel(uint4* __restrict__ out,
                                                                   long long n16)
{
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u < n16) out[u] = make_uint4((uint32_t)u, (uint32_t)(u >> 32), 0u, 0u);
}

// workgroup b reads the 16-byte units [b * blockDim, (b + 1) * blockDim) of in and folds them
// into one word; a word is stored only when it equals a sentinel, which keeps the loads live
__global__ __launch_bounds__(1024) void ceiling_read_chunks_kernel(const uint4* __restrict__ in,
                                                                  uint32_t* __restrict__ sink,
                                                                  long long n16)
{
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    if (u < n16) {
        const uint4 v = load_nt(in + u);
        acc = v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// x bf16 [T][H]; rows int32 [T][K] (a destination row per pick, -1 for none); out [rows][H]
// bytes.  H a multiple of 1024, at most 8192; K at most 16.  Returns a hipError_t value.
int ceiling_scatter_copy(const void* x, const int32_t* rows, void* out, long long T, int H,
                         int K, void* stream)
{
    if (H % 1024 != 0 || H > 8192 || K < 1 || K > kMaxK) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(ceiling_scatter_copy_kernel, dim3((unsigned)T), dim3(H / 16), 0,
                       (hipStream_t)stream, static_cast<const uint16_t*>(x), rows,
                       static_cast<uint8_t*>(out), H, K);
    return (int)hipGetLastError();
}

// out [rows][H] bytes; order int32 [rows] (a permutation of [0, rows)) or NULL for sequence.
int ceiling_write_rows(void* out, const int32_t* order, long long rows, int H, void* stream)
{
    if (H % 8 != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(ceiling_write_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, static_cast<uint8_t*>(out), order, rows, H);
    return (int)hipGetLastError();
}

// rows bf16 [.][H]; src int32 [T][K] (the source row of each pick, or -1); y bf16 [T][H].
// H a multiple of 8; K at most 16.
int ceiling_gather_sum(const void* rows, const int32_t* src, void* y, long long T, int H, int K,
                       void* stream)
{
    if (H % 8 != 0 || K < 1 || K > kMaxK) return (int)hipErrorInvalidValue;
    const int tasks_per_token = (H / 8 + 2 * kWave - 1) / (2 * kWave);
    const long long tasks = T * tasks_per_token;
    const unsigned blocks = (unsigned)((tasks + 3) / 4);
#define MOE_DC_GATHER(KM)                                                                    \
    hipLaunchKernelGGL((ceiling_gather_sum_kernel<KM>), dim3(blocks), dim3(256), 0,           \
                       (hipStream_t)stream, static_cast<const uint4*>(rows), src,            \
                       static_cast<uint4*>(y), T, H, K, tasks_per_token)
    if (K <= 8) MOE_DC_GATHER(8);
    else MOE_DC_GATHER(16);
#undef MOE_DC_GATHER
    return (int)hipGetLastError();
}

// out: bytes (a multiple of 16) bytes, 16-byte aligned; chunk: bytes per workgroup, a multiple
// of 1024 up to 16384 (one wave per KiB).
int ceiling_write_chunks(void* out, long long bytes, int chunk, void* stream)
{
    if (bytes % 16 != 0 || bytes <= 0 || chunk % 1024 != 0 || chunk < 1024 || chunk > 16384)
        return (int)hipErrorInvalidValue;
    const long long n16 = bytes / 16;
    const int lanes = chunk / 16;
    hipLaunchKernelGGL(ceiling_write_chunks_kernel, dim3((unsigned)((n16 + lanes - 1) / lanes)),
                       dim3(lanes), 0, (hipStream_t)stream, static_cast<uint4*>(out), n16);
    return (int)hipGetLastError();
}

// in: bytes (a multiple of 16) bytes, 16-byte aligned; sink: 1024 words; chunk as above.
int ceiling_read_chunks(const void* in, void* sink, long long bytes, int chunk, void* stream)
{
    if (bytes % 16 != 0 || bytes <= 0 || chunk % 1024 != 0 || chunk < 1024 || chunk > 16384)
        return (int)hipErrorInvalidValue;
    const long long n16 = bytes / 16;
    const int lanes = chunk / 16;
    hipLaunchKernelGGL(ceiling_read_chunks_kernel, dim3((unsigned)((n16 + lanes - 1) / lanes)),
                       dim3(lanes), 0, (hipStream_t)stream, static_cast<const uint4*>(in),
                       static_cast<uint32_t*>(sink), n16);
    return (int)hipGetLastError();
}

}  // extern "C"
