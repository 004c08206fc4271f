/*
 * The linear layer called from C through include/mxfp.h alone: no Python in the call path.
 *
 *   linear_from_c A.bin W.bin BIAS.bin OUT.bin M K N
 *
 * A.bin: M x K BF16 bit patterns (row-major), W.bin: N x K BF16, BIAS.bin: N FP16, all little
 * endian.  The weight is quantized to MXFP4 in the tiled layout (mx_quantize), then
 * mx_linear quantizes A dynamically and multiplies, with the bias epilogue and FP32 output.
 * OUT.bin receives M x N float32 values.  Exit status 0 on success; a failing call prints its
 * status name and mx_last_error().
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mxfp.h"

static void* read_file(const char* path, size_t bytes) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

#define HIP_CHECK(call)                                                               \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

#define MX_CHECK(call)                                                                        \
    do {                                                                                      \
        mx_status s_ = (call);                                                                \
        if (s_ != MX_OK) {                                                                    \
            fprintf(stderr, "%s: %s (%s)\n", #call, mx_status_string(s_), mx_last_error());   \
            return 3;                                                                         \
        }                                                                                     \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 8) {
        fprintf(stderr, "usage: %s A.bin W.bin BIAS.bin OUT.bin M K N\n", argv[0]);
        return 1;
    }
    const int64_t M = atoll(argv[5]), K = atoll(argv[6]), N = atoll(argv[7]);
    if (M <= 0 || K <= 0 || N <= 0 || K % 128) {
        fprintf(stderr, "need M, K, N > 0 and K %% 128 == 0\n");
        return 1;
    }
    uint16_t* ha = read_file(argv[1], (size_t)(M * K * 2));
    uint16_t* hw = read_file(argv[2], (size_t)(N * K * 2));
    uint16_t* hb = read_file(argv[3], (size_t)(N * 2));
    float* hy = malloc((size_t)(M * N * 4));
    if (!ha || !hw || !hb || !hy) {
        fprintf(stderr, "cannot read the input files\n");
        return 1;
    }
    if (mx_abi_version() != MX_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header %d\n", mx_abi_version(), MX_ABI_VERSION);
        return 1;
    }

    size_t wc_bytes = 0, ws_bytes = 0;
    MX_CHECK(mx_tiled_bytes(N, K, MX_FMT_MXFP4, &wc_bytes, &ws_bytes));
    const size_t work_bytes = mx_linear_workspace_bytes(M, K, MX_FMT_MXFP4, 0);

    void *da, *dw, *db, *dy, *dwc, *dws, *dwork;
    HIP_CHECK(hipMalloc(&da, (size_t)(M * K * 2)));
    HIP_CHECK(hipMalloc(&dw, (size_t)(N * K * 2)));
    HIP_CHECK(hipMalloc(&db, (size_t)(N * 2)));
    HIP_CHECK(hipMalloc(&dy, (size_t)(M * N * 4)));
    HIP_CHECK(hipMalloc(&dwc, wc_bytes));
    HIP_CHECK(hipMalloc(&dws, ws_bytes));
    HIP_CHECK(hipMalloc(&dwork, work_bytes ? work_bytes : 1));
    HIP_CHECK(hipMemcpy(da, ha, (size_t)(M * K * 2), hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dw, hw, (size_t)(N * K * 2), hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(db, hb, (size_t)(N * 2), hipMemcpyHostToDevice));

    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    /* offline weight preparation, then the layer itself */
    MX_CHECK(mx_quantize((const uint16_t*)dw, N, K, K, MX_FMT_MXFP4, MX_LAYOUT_TILED, 1.0f, dwc,
                         (uint8_t*)dws, stream));
    const mx_qmatrix w = {dwc, (const uint8_t*)dws, 1.0f, MX_FMT_MXFP4, N, K, MX_LAYOUT_TILED};
    MX_CHECK(mx_linear((const uint16_t*)da, M, K, K, MX_FMT_MXFP4, 1.0f, &w, (const uint16_t*)db, NULL,
                       MX_EPI_BIAS, MX_OUT_F32, dy, N, NULL, dwork, work_bytes, stream));
    HIP_CHECK(hipStreamSynchronize(stream));
    HIP_CHECK(hipMemcpy(hy, dy, (size_t)(M * N * 4), hipMemcpyDeviceToHost));

    FILE* f = fopen(argv[4], "wb");
    if (!f || fwrite(hy, 4, (size_t)(M * N), f) != (size_t)(M * N)) {
        fprintf(stderr, "cannot write %s\n", argv[4]);
        return 1;
    }
    fclose(f);
    hipStreamDestroy(stream);
    hipFree(da), hipFree(dw), hipFree(db), hipFree(dy), hipFree(dwc), hipFree(dws), hipFree(dwork);
    free(ha), free(hw), free(hb), free(hy);
    printf("linear_from_c: %lld x %lld x %lld ok\n", (long long)M, (long long)K, (long long)N);
    return 0;
}
