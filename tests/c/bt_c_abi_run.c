/*
 * A plain C caller of libbt: no Python, no torch. It reads one projection's
 * inputs from a file, runs the library's path through the C ABI alone
 * (host pack, device repack, per-token quantization, ternary matmul, and for
 * M <= BT_GEMV_MAX_M the fused call) with hipMalloc'd buffers on one stream,
 * and writes every output to a file, which the test compares with the CPU
 * oracle. It holds none of the method's arithmetic.
 *
 * Input file (little-endian): int64 M, N, K; float w_scale; then M*K fp32 x
 * (row-major), then N*K int8 w (row-major, values in {-1, 0, 1}).
 * Output file: the status of every call as int32 (pack, repack, quantize,
 * matmul, fused; the fused one BT_OK when skipped), then M*K int8 q,
 * M fp32 xscale, M int32 xsum, M*N int32 acc, M*N fp32 y, and for the
 * fused call M*K int8 q, M fp32 xscale, M int32 xsum, M*N int32 acc,
 * M*N fp32 y (zeros when skipped).
 *
 * Exit status: 0 when every call returned BT_OK and every HIP call
 * succeeded, 1 otherwise (the output file is written either way when it can
 * be).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bt.h"

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    if (bytes == 0) return NULL;
    HIP_OK(hipMalloc(&p, bytes));
    return p;
}

static void read_exact(FILE* f, void* dst, size_t bytes) {
    if (fread(dst, 1, bytes, f) != bytes) {
        fprintf(stderr, "short input file\n");
        exit(1);
    }
}

static void write_all(FILE* f, const void* src, size_t bytes) {
    if (fwrite(src, 1, bytes, f) != bytes) {
        fprintf(stderr, "short write\n");
        exit(1);
    }
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s input output\n", argv[0]);
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) {
        perror(argv[1]);
        return 1;
    }
    int64_t dims[3];
    float w_scale;
    read_exact(in, dims, sizeof(dims));
    read_exact(in, &w_scale, sizeof(w_scale));
    const int64_t M = dims[0], N = dims[1], K = dims[2];
    if (M < 1 || N < 1 || K < 1 || M * K > (1 << 26) || N * K > (1 << 28) || M * N > (1 << 26)) {
        fprintf(stderr, "shape out of this program's range\n");
        return 1;
    }
    float* x = malloc((size_t)(M * K) * sizeof(float));
    int8_t* w = malloc((size_t)(N * K));
    read_exact(in, x, (size_t)(M * K) * sizeof(float));
    read_exact(in, w, (size_t)(N * K));
    fclose(in);

    int32_t status[5] = {0, 0, 0, 0, BT_OK};
    const size_t packed_bytes = bt_packed_bytes(N, K);
    const size_t repacked_bytes = bt_repacked_bytes(N, K);
    uint8_t* packed = malloc(packed_bytes ? packed_bytes : 1);
    status[0] = bt_pack_ternary(w, N, K, packed);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    uint8_t* d_packed = dev_alloc(packed_bytes);
    void* d_w = dev_alloc(repacked_bytes);
    float* d_x = dev_alloc((size_t)(M * K) * sizeof(float));
    int8_t* d_q = dev_alloc((size_t)(M * K));
    float* d_xs = dev_alloc((size_t)M * sizeof(float));
    int32_t* d_xsum = dev_alloc((size_t)M * sizeof(int32_t));
    int32_t* d_acc = dev_alloc((size_t)(M * N) * sizeof(int32_t));
    float* d_y = dev_alloc((size_t)(M * N) * sizeof(float));
    const size_t ws_bytes = bt_matmul_workspace_bytes(M, N, K);
    void* d_ws = dev_alloc(ws_bytes);
    HIP_OK(hipMemcpyAsync(d_packed, packed, packed_bytes, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(d_x, x, (size_t)(M * K) * sizeof(float), hipMemcpyHostToDevice, stream));

    status[1] = bt_repack_ternary(d_packed, N, K, d_w, stream);
    status[2] = bt_quantize_act(d_x, M, K, d_q, d_xs, d_xsum, stream);
    status[3] = bt_ternary_matmul(M, N, K, d_q, d_xs, d_xsum, d_w, w_scale, d_y, d_acc, d_ws,
                                  ws_bytes, stream);

    const size_t nq = (size_t)(M * K), ny = (size_t)(M * N);
    int8_t* q = calloc(nq, 1);
    float* xs = calloc((size_t)M, sizeof(float));
    int32_t* xsum = calloc((size_t)M, sizeof(int32_t));
    int32_t* acc = calloc(ny, sizeof(int32_t));
    float* y = calloc(ny, sizeof(float));
    int8_t* fq = calloc(nq, 1);
    float* fxs = calloc((size_t)M, sizeof(float));
    int32_t* fxsum = calloc((size_t)M, sizeof(int32_t));
    int32_t* facc = calloc(ny, sizeof(int32_t));
    float* fy = calloc(ny, sizeof(float));
    HIP_OK(hipMemcpyAsync(q, d_q, nq, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(xs, d_xs, (size_t)M * sizeof(float), hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(xsum, d_xsum, (size_t)M * sizeof(int32_t), hipMemcpyDeviceToHost,
                          stream));
    HIP_OK(hipMemcpyAsync(acc, d_acc, ny * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(y, d_y, ny * sizeof(float), hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));

    if (M <= BT_GEMV_MAX_M) {
        /* the fused call writes fresh buffers: clear them first */
        HIP_OK(hipMemsetAsync(d_q, 0, nq, stream));
        HIP_OK(hipMemsetAsync(d_xs, 0, (size_t)M * sizeof(float), stream));
        HIP_OK(hipMemsetAsync(d_xsum, 0, (size_t)M * sizeof(int32_t), stream));
        HIP_OK(hipMemsetAsync(d_acc, 0, ny * sizeof(int32_t), stream));
        HIP_OK(hipMemsetAsync(d_y, 0, ny * sizeof(float), stream));
        status[4] = bt_ternary_matmul_fused(M, N, K, d_x, d_w, w_scale, d_y, d_acc, d_q, d_xs,
                                            d_xsum, d_ws, ws_bytes, stream);
        HIP_OK(hipMemcpyAsync(fq, d_q, nq, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipMemcpyAsync(fxs, d_xs, (size_t)M * sizeof(float), hipMemcpyDeviceToHost,
                              stream));
        HIP_OK(hipMemcpyAsync(fxsum, d_xsum, (size_t)M * sizeof(int32_t), hipMemcpyDeviceToHost,
                              stream));
        HIP_OK(hipMemcpyAsync(facc, d_acc, ny * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
        HIP_OK(hipMemcpyAsync(fy, d_y, ny * sizeof(float), hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));
    }

    FILE* out = fopen(argv[2], "wb");
    if (!out) {
        perror(argv[2]);
        return 1;
    }
    write_all(out, status, sizeof(status));
    write_all(out, q, nq);
    write_all(out, xs, (size_t)M * sizeof(float));
    write_all(out, xsum, (size_t)M * sizeof(int32_t));
    write_all(out, acc, ny * sizeof(int32_t));
    write_all(out, y, ny * sizeof(float));
    write_all(out, fq, nq);
    write_all(out, fxs, (size_t)M * sizeof(float));
    write_all(out, fxsum, (size_t)M * sizeof(int32_t));
    write_all(out, facc, ny * sizeof(int32_t));
    write_all(out, fy, ny * sizeof(float));
    fclose(out);

    int ok = 1;
    for (int i = 0; i < 5; ++i) {
        if (status[i] != BT_OK) {
            fprintf(stderr, "call %d: %s\n", i, bt_status_string((bt_status)status[i]));
            ok = 0;
        }
    }
    HIP_OK(hipFree(d_packed));
    HIP_OK(hipFree(d_w));
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_q));
    HIP_OK(hipFree(d_xs));
    HIP_OK(hipFree(d_xsum));
    HIP_OK(hipFree(d_acc));
    HIP_OK(hipFree(d_y));
    if (d_ws) HIP_OK(hipFree(d_ws));
    HIP_OK(hipStreamDestroy(stream));
    free(x);
    free(w);
    free(packed);
    free(q);
    free(xs);
    free(xsum);
    free(acc);
    free(y);
    free(fq);
    free(fxs);
    free(fxsum);
    free(facc);
    free(fy);
    return ok ? 0 : 1;
}
