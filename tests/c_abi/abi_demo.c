/*
 * abi_demo.c -- a plain C11 consumer of libmoe_dc (include/moe_dc.h), linked against the HIP
 * runtime only: no Python, no C++.  It checks the library end to end with invariants that
 * need no reference implementation, then times dispatch + combine launched from native code.
 *
 * usage: abi_demo W E BS H K iters
 *
 * Inputs: x[s][i][h] = small integers / 64 (exact in bf16); each token picks K distinct experts
 * (a seeded linear congruential generator); weights 1/K with K a power of two.  Dispatch runs
 * without quantization, so the identity "expert" is expand_x itself, and the combine of K
 * copies of x weighted 1/K must return x bit for bit.
 * Checks: every status is MOE_OK; recv_offsets[W] = W*BS*K (nothing masked, no special
 * experts) = the sum of expert_token_nums (type 1); every expand_x row holds the bf16 row of
 * the token its assist_info triple names, and every pick appears exactly once; y == x.
 * The other two combines run on the same rows: the scatter-back combine (moe_combine_scatter,
 * rows returned by their triples) must also give x bit for bit, and the int8 block-quantized
 * combine (moe_combine_quantize, then moe_combine_int8) x within its quantization bound:
 * 0.6 * (the 8-element block's max |x|) / 127 plus the bf16 rounding of the result.  The
 * dispatch for callers that cannot allocate (moe_dispatch_no_workspace) must give the same
 * bytes as moe_dispatch in every output.
 * Prints "ok routed=<rows> step_us=<mean>" and exits 0, or prints the failure and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_dc.h"

#define HIP_OK(call)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            printf("hip error %s at line %d\n", hipGetErrorString(e_), __LINE__);        \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

#define MOE_OK_OR_FAIL(call)                                                              \
    do {                                                                                  \
        moe_status st_ = (call);                                                          \
        if (st_ != MOE_OK) {                                                              \
            printf("moe status %d at line %d: %s\n", (int)st_, __LINE__, moe_dc_last_error()); \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

static uint32_t lcg_state = 12345u;
static uint32_t lcg(void)
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return lcg_state >> 8;
}

/* bf16 pattern of a float that bf16 holds exactly (the low 16 bits are zero) */
static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static float f32_of_bf16(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int main(int argc, char** argv)
{
    if (argc != 7) {
        printf("usage: abi_demo W E BS H K iters\n");
        return 1;
    }
    const int W = atoi(argv[1]), E = atoi(argv[2]), BS = atoi(argv[3]), H = atoi(argv[4]);
    const int K = atoi(argv[5]), iters = atoi(argv[6]);
    if ((K & (K - 1)) != 0 || K > E) {
        printf("K must be a power of two and at most E\n");
        return 1;
    }
    moe_dc_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.ep_world_size = W;
    cfg.moe_expert_num = E;
    cfg.bs = BS;
    cfg.hidden = H;
    cfg.topk = K;
    cfg.quant_mode = 0;
    cfg.expert_token_nums_type = 1;
    cfg.expand_rows_capacity = (int64_t)W * BS * K;
    MOE_OK_OR_FAIL(moe_dc_validate(&cfg));
    const size_t T = (size_t)W * BS, cap = (size_t)cfg.expand_rows_capacity, L = (size_t)E / W;
    const size_t ws_bytes = moe_dc_dispatch_workspace_bytes(&cfg);
    if (ws_bytes == 0 || moe_dc_scales_per_row(&cfg) != 0) {
        printf("unexpected workspace or scale count\n");
        return 1;
    }

    uint16_t* x = malloc(T * H * sizeof(uint16_t));
    int32_t* ids = malloc(T * K * sizeof(int32_t));
    float* w = malloc(T * K * sizeof(float));
    for (size_t n = 0; n < T * H; ++n) x[n] = bf16_of((float)((int)(lcg() % 2001) - 1000) / 64.0f);
    for (size_t t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e, dup;
            do {                                       /* K distinct experts per token */
                e = (int)(lcg() % (uint32_t)E);
                dup = 0;
                for (int j = 0; j < k; ++j) dup |= ids[t * K + j] == e;
            } while (dup);
            ids[t * K + k] = e;
            w[t * K + k] = 1.0f / (float)K;
        }

    void *dx, *dids, *dw, *dex, *deidx, *dai, *derc, *detn, *droff, *dws, *dy;
    HIP_OK(hipMalloc(&dx, T * H * 2));
    HIP_OK(hipMalloc(&dids, T * K * 4));
    HIP_OK(hipMalloc(&dw, T * K * 4));
    HIP_OK(hipMalloc(&dex, cap * H * 2));
    HIP_OK(hipMalloc(&deidx, T * K * 4));
    HIP_OK(hipMalloc(&dai, cap * 3 * 4));
    HIP_OK(hipMalloc(&derc, (size_t)W * L * W * 4));
    HIP_OK(hipMalloc(&detn, (size_t)W * L * 8));
    HIP_OK(hipMalloc(&droff, (size_t)(W + 1) * 8));
    HIP_OK(hipMalloc(&dws, ws_bytes));
    HIP_OK(hipMalloc(&dy, T * H * 2));
    HIP_OK(hipMemcpy(dx, x, T * H * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dids, ids, T * K * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw, w, T * K * 4, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* one round trip, checked */
    MOE_OK_OR_FAIL(moe_dispatch(&cfg, dx, dids, NULL, NULL, NULL, dex, NULL, deidx, dai, derc,
                                detn, droff, NULL, dws, ws_bytes, stream));
    MOE_OK_OR_FAIL(moe_combine(&cfg, dex, dids, deidx, dw, derc, droff, NULL, NULL, dy, stream));
    HIP_OK(hipStreamSynchronize(stream));

    int64_t* roff = malloc((size_t)(W + 1) * 8);
    int64_t* etn = malloc((size_t)W * L * 8);
    int32_t* ai = malloc(cap * 3 * 4);
    uint16_t* ex = malloc(cap * H * 2);
    uint16_t* y = malloc(T * H * 2);
    HIP_OK(hipMemcpy(roff, droff, (size_t)(W + 1) * 8, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(etn, detn, (size_t)W * L * 8, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ai, dai, cap * 3 * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ex, dex, cap * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, dy, T * H * 2, hipMemcpyDeviceToHost));

    const int64_t P = roff[W];
    int64_t etn_sum = 0;
    for (size_t n = 0; n < (size_t)W * L; ++n) etn_sum += etn[n];
    if (P != (int64_t)(T * K) || etn_sum != P) {
        printf("routed rows %lld, expert_token_nums sum %lld, want %zu\n", (long long)P,
               (long long)etn_sum, T * K);
        return 1;
    }
    unsigned char* seen = calloc(T * K, 1);
    for (int64_t r = 0; r < P; ++r) {
        const int s = ai[r * 3], i = ai[r * 3 + 1], k = ai[r * 3 + 2];
        if (s < 0 || s >= W || i < 0 || i >= BS || k < 0 || k >= K) {
            printf("row %lld: bad triple\n", (long long)r);
            return 1;
        }
        const size_t p = ((size_t)s * BS + i) * K + k;
        if (seen[p]++) {
            printf("pick %zu stored twice\n", p);
            return 1;
        }
        if (memcmp(ex + (size_t)r * H, x + ((size_t)s * BS + i) * H, (size_t)H * 2) != 0) {
            printf("row %lld does not hold its token\n", (long long)r);
            return 1;
        }
    }
    if (memcmp(y, x, T * H * 2) != 0) {
        printf("combine of K copies weighted 1/K is not x\n");
        return 1;
    }

    /* scatter-back combine: the rows go back by their triples; the same sum in k order */
    const size_t ws2_bytes = moe_dc_combine_scatter_workspace_bytes(&cfg);
    void *dws2, *dy2, *dcodes, *dbs, *dy3;
    const size_t nb = ((size_t)H + 7) / 8;
    HIP_OK(hipMalloc(&dws2, ws2_bytes));
    HIP_OK(hipMalloc(&dy2, T * H * 2));
    HIP_OK(hipMalloc(&dcodes, cap * H));
    HIP_OK(hipMalloc(&dbs, cap * nb * 4));
    HIP_OK(hipMalloc(&dy3, T * H * 2));
    MOE_OK_OR_FAIL(moe_combine_scatter(&cfg, dex, dai, droff, dids, dw, NULL, NULL, NULL, dy2,
                                       dws2, ws2_bytes, stream));
    /* int8 block-quantized combine over the same rows */
    MOE_OK_OR_FAIL(moe_combine_quantize(&cfg, dex, droff, dcodes, dbs, stream));
    MOE_OK_OR_FAIL(moe_combine_int8(&cfg, dcodes, dbs, dids, deidx, dw, derc, droff, NULL, NULL,
                                    dy3, stream));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(y, dy2, T * H * 2, hipMemcpyDeviceToHost));
    if (memcmp(y, x, T * H * 2) != 0) {
        printf("scatter-back combine of K copies weighted 1/K is not x\n");
        return 1;
    }
    HIP_OK(hipMemcpy(y, dy3, T * H * 2, hipMemcpyDeviceToHost));
    for (size_t t = 0; t < T; ++t)
        for (size_t b0 = 0; b0 < (size_t)H; b0 += 8) {
            float amax = 0.0f;
            for (size_t h = b0; h < b0 + 8 && h < (size_t)H; ++h) {
                const float a = f32_of_bf16(x[t * H + h]);
                amax = a > amax ? a : (-a > amax ? -a : amax);
            }
            for (size_t h = b0; h < b0 + 8 && h < (size_t)H; ++h) {
                const float xv = f32_of_bf16(x[t * H + h]), yv = f32_of_bf16(y[t * H + h]);
                const float d = yv > xv ? yv - xv : xv - yv;
                const float ax = xv > 0.0f ? xv : -xv;
                if (d > 0.6f * amax / 127.0f + ax / 256.0f + 1e-6f) {
                    printf("int8 combine: token %zu element %zu: %g vs %g\n", t, h, yv, xv);
                    return 1;
                }
            }
        }

    /* the dispatch for callers that cannot allocate (its workspace is the library's static
     * device array): every output the same bytes as moe_dispatch's */
    {
        int32_t* eidx = malloc(T * K * 4);
        int32_t* erc = malloc((size_t)W * L * W * 4);
        int32_t* eidx2 = malloc(T * K * 4);
        int32_t* erc2 = malloc((size_t)W * L * W * 4);
        int64_t* etn2 = malloc((size_t)W * L * 8);
        int64_t* roff2 = malloc((size_t)(W + 1) * 8);
        int32_t* ai2 = malloc(cap * 3 * 4);
        uint16_t* ex2 = malloc(cap * H * 2);
        void *dex2, *deidx2, *dai2, *derc2, *detn2, *droff2;
        HIP_OK(hipMemcpy(eidx, deidx, T * K * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(erc, derc, (size_t)W * L * W * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMalloc(&dex2, cap * H * 2));
        HIP_OK(hipMalloc(&deidx2, T * K * 4));
        HIP_OK(hipMalloc(&dai2, cap * 3 * 4));
        HIP_OK(hipMalloc(&derc2, (size_t)W * L * W * 4));
        HIP_OK(hipMalloc(&detn2, (size_t)W * L * 8));
        HIP_OK(hipMalloc(&droff2, (size_t)(W + 1) * 8));
        MOE_OK_OR_FAIL(moe_dispatch_no_workspace(&cfg, dx, dids, NULL, NULL, NULL, dex2, NULL,
                                                 deidx2, dai2, derc2, detn2, droff2, NULL,
                                                 stream));
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(eidx2, deidx2, T * K * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(erc2, derc2, (size_t)W * L * W * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(etn2, detn2, (size_t)W * L * 8, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(roff2, droff2, (size_t)(W + 1) * 8, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ai2, dai2, cap * 3 * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ex2, dex2, cap * H * 2, hipMemcpyDeviceToHost));
        if (memcmp(eidx, eidx2, T * K * 4) != 0 || memcmp(erc, erc2, (size_t)W * L * W * 4) != 0 ||
            memcmp(etn, etn2, (size_t)W * L * 8) != 0 ||
            memcmp(roff, roff2, (size_t)(W + 1) * 8) != 0 ||
            memcmp(ai, ai2, (size_t)P * 3 * 4) != 0 || memcmp(ex, ex2, (size_t)P * H * 2) != 0) {
            printf("moe_dispatch_no_workspace differs from moe_dispatch\n");
            return 1;
        }
        HIP_OK(hipFree(dex2));
        HIP_OK(hipFree(deidx2));
        HIP_OK(hipFree(dai2));
        HIP_OK(hipFree(derc2));
        HIP_OK(hipFree(detn2));
        HIP_OK(hipFree(droff2));
        free(eidx); free(erc); free(eidx2); free(erc2); free(etn2); free(roff2); free(ai2);
        free(ex2);
    }

    /* native launch timing: dispatch + combine, eager, on one stream */
    hipEvent_t a, b;
    HIP_OK(hipEventCreate(&a));
    HIP_OK(hipEventCreate(&b));
    for (int n = 0; n < 3; ++n) {
        MOE_OK_OR_FAIL(moe_dispatch(&cfg, dx, dids, NULL, NULL, NULL, dex, NULL, deidx, dai,
                                    derc, detn, droff, NULL, dws, ws_bytes, stream));
        MOE_OK_OR_FAIL(moe_combine(&cfg, dex, dids, deidx, dw, derc, droff, NULL, NULL, dy,
                                   stream));
    }
    HIP_OK(hipEventRecord(a, stream));
    for (int n = 0; n < iters; ++n) {
        MOE_OK_OR_FAIL(moe_dispatch(&cfg, dx, dids, NULL, NULL, NULL, dex, NULL, deidx, dai,
                                    derc, detn, droff, NULL, dws, ws_bytes, stream));
        MOE_OK_OR_FAIL(moe_combine(&cfg, dex, dids, deidx, dw, derc, droff, NULL, NULL, dy,
                                   stream));
    }
    HIP_OK(hipEventRecord(b, stream));
    HIP_OK(hipEventSynchronize(b));
    float ms = 0.0f;
    HIP_OK(hipEventElapsedTime(&ms, a, b));
    printf("ok routed=%lld step_us=%.2f version=%s\n", (long long)P, 1000.0f * ms / iters,
           moe_dc_version());
    return 0;
}
