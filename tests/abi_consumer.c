/*
 * A plain C99 program that uses libskipln through include/skipln.h alone:
 * HIP runtime calls for memory and a stream, the operator's entry points for
 * the work.  No Python, no torch.  The GPU test writes the tensors to files,
 * runs this program, and compares what it writes back with the oracle.
 *
 * usage: abi_consumer DIR rows hidden dtype skip_rows has_beta has_bias
 *                     has_residual eps
 *   DIR holds input.bin, skip.bin, gamma.bin and, when present, beta.bin and
 *   bias.bin (raw little-endian elements of dtype: 0 float32, 1 float16);
 *   skip_rows 0 = exact skip, else the broadcast skip's row count.
 *   Writes DIR/out.bin and, with has_residual, DIR/residual.bin.
 *
 * Besides the result, it checks the status codes of rejected arguments, that
 * skipln_validate agrees with skipln_forward, that the no-allocation entry
 * point gives the same bytes as the workspace form, and that both give
 * skipln_forward's bytes when the call needs no workspace.
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "skipln.h"

#define FAIL(...)                                   \
    do {                                            \
        fprintf(stderr, "abi_consumer: " __VA_ARGS__); \
        fputc('\n', stderr);                        \
        exit(1);                                    \
    } while (0)

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) FAIL("%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

#define EXPECT_STATUS(call, want)                                                        \
    do {                                                                                 \
        int s_ = (call);                                                                 \
        if (s_ != (want)) FAIL("%s returned %d (%s), expected %d", #call, s_,           \
                               skipln_status_string(s_), (int)(want));                    \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) FAIL("cannot open %s", path);
    void* p = malloc(bytes ? bytes : 1);
    if (!p) FAIL("out of host memory");
    if (fread(p, 1, bytes, f) != bytes) FAIL("%s holds fewer than %zu bytes", path, bytes);
    fclose(f);
    return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) FAIL("cannot write %s", path);
    fclose(f);
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void* from_device(const void* dev, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h) FAIL("out of host memory");
    if (bytes) HIP_OK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    return h;
}

int main(int argc, char** argv) {
    if (argc != 10) FAIL("usage: abi_consumer DIR rows hidden dtype skip_rows has_beta has_bias has_residual eps");
    const char* dir = argv[1];
    const int64_t rows = strtoll(argv[2], NULL, 10);
    const int64_t hidden = strtoll(argv[3], NULL, 10);
    const int dtype = atoi(argv[4]);
    const int64_t skip_rows = strtoll(argv[5], NULL, 10);
    const int has_beta = atoi(argv[6]), has_bias = atoi(argv[7]), has_res = atoi(argv[8]);
    const float eps = strtof(argv[9], NULL);
    const int mode = skip_rows > 0 ? SKIPLN_SKIP_BROADCAST : SKIPLN_SKIP_EXACT;
    const size_t es = dtype == SKIPLN_F32 ? 4 : 2;
    const size_t nx = (size_t)rows * (size_t)hidden * es;
    const size_t ns = (size_t)(skip_rows > 0 ? skip_rows : rows) * (size_t)hidden * es;
    const size_t nv = (size_t)hidden * es;

    if (skipln_version() != 2) FAIL("skipln_version() = %d, this program is written for 2", skipln_version());

    void* h_x = read_file(dir, "input.bin", nx);
    void* h_s = read_file(dir, "skip.bin", ns);
    void* h_g = read_file(dir, "gamma.bin", nv);
    void* h_b = has_beta ? read_file(dir, "beta.bin", nv) : NULL;
    void* h_bias = has_bias ? read_file(dir, "bias.bin", nv) : NULL;

    void* x = to_device(h_x, nx);
    void* s = to_device(h_s, ns);
    void* g = to_device(h_g, nv);
    void* b = has_beta ? to_device(h_b, nv) : NULL;
    void* bias = has_bias ? to_device(h_bias, nv) : NULL;
    void *out = NULL, *out_ws = NULL, *out_static = NULL, *res = NULL;
    HIP_OK(hipMalloc(&out, nx ? nx : 16));
    HIP_OK(hipMalloc(&out_ws, nx ? nx : 16));
    HIP_OK(hipMalloc(&out_static, nx ? nx : 16));
    if (has_res) HIP_OK(hipMalloc(&res, nx ? nx : 16));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* Host-only checks agree with the call. */
    EXPECT_STATUS(skipln_validate(x, s, mode, skip_rows, g, b, bias, out, res, rows, hidden, eps, dtype), SKIPLN_OK);
    EXPECT_STATUS(skipln_validate(x, s, mode, skip_rows, NULL, b, bias, out, res, rows, hidden, eps, dtype),
                  SKIPLN_ERR_NULL);

    /* Rejected arguments enqueue nothing and name their fault. */
    EXPECT_STATUS(skipln_forward(x, s, mode, skip_rows, NULL, b, bias, out, res, rows, hidden, eps, dtype, stream),
                  SKIPLN_ERR_NULL);
    EXPECT_STATUS(skipln_forward(x, s, mode, skip_rows, g, b, bias, out, res, rows, hidden, -1.0f, dtype, stream),
                  SKIPLN_ERR_EPS);
    EXPECT_STATUS(skipln_forward(x, s, mode, skip_rows, g, b, bias, out, res, rows, hidden, eps, 7, stream),
                  SKIPLN_ERR_DTYPE);
    EXPECT_STATUS(skipln_forward(x, s, 9, skip_rows, g, b, bias, out, res, rows, hidden, eps, dtype, stream),
                  SKIPLN_ERR_MODE);
    EXPECT_STATUS(skipln_forward(x, s, mode, skip_rows, g, b, bias, out, res, rows, 0, eps, dtype, stream),
                  SKIPLN_ERR_SHAPE);
    if (rows > 1)
        EXPECT_STATUS(skipln_forward(x, s, mode, skip_rows, g, b, bias, (char*)x + es, res, rows, hidden, eps, dtype,
                                     stream),
                      SKIPLN_ERR_ALIAS);
    for (int st = 0; st <= SKIPLN_ERR_WORKSPACE; ++st) {
        const char* msg = skipln_status_string(st);
        if (!msg || !msg[0]) FAIL("skipln_status_string(%d) is empty", st);
    }

    /* The operator, then the same call through the workspace and the
     * no-allocation entry points. */
    EXPECT_STATUS(skipln_forward(x, s, mode, skip_rows, g, b, bias, out, res, rows, hidden, eps, dtype, stream),
                  SKIPLN_OK);
    const int64_t ws_bytes = skipln_workspace_bytes(SKIPLN_OP_LAYER_NORM, rows, hidden, dtype, mode, skip_rows);
    if (ws_bytes < 0) FAIL("skipln_workspace_bytes returned %lld", (long long)ws_bytes);
    void* ws = NULL;
    if (ws_bytes > 0) HIP_OK(hipMalloc(&ws, (size_t)ws_bytes));
    EXPECT_STATUS(skipln_forward_ws(SKIPLN_OP_LAYER_NORM, x, s, mode, skip_rows, g, b, bias, out_ws, NULL, rows, hidden,
                                    eps, dtype, ws, ws_bytes, stream),
                  SKIPLN_OK);
    EXPECT_STATUS(skipln_forward_ws_static(SKIPLN_OP_LAYER_NORM, x, s, mode, skip_rows, g, b, bias, out_static, NULL,
                                           rows, hidden, eps, dtype, stream),
                  SKIPLN_OK);
    HIP_OK(hipStreamSynchronize(stream));

    void* h_out = from_device(out, nx);
    void* h_out_ws = from_device(out_ws, nx);
    void* h_out_static = from_device(out_static, nx);
    /* With a workspace the automatic choice may split long rows across
     * workgroups (a different summation order); without one it runs the same
     * kernels as skipln_forward.  The no-allocation entry point always
     * matches the workspace form. */
    if (ws_bytes == 0 && memcmp(h_out, h_out_ws, nx) != 0)
        FAIL("skipln_forward_ws output differs from skipln_forward's");
    if (memcmp(h_out_ws, h_out_static, nx) != 0) FAIL("skipln_forward_ws_static output differs from skipln_forward_ws's");
    write_file(dir, "out.bin", h_out, nx);
    if (has_res) {
        void* h_res = from_device(res, nx);
        write_file(dir, "residual.bin", h_res, nx);
        free(h_res);
    }
    printf("abi_consumer: rows=%lld hidden=%lld dtype=%d skip_rows=%lld workspace=%lld ok\n", (long long)rows,
           (long long)hidden, dtype, (long long)skip_rows, (long long)ws_bytes);

    HIP_OK(hipStreamDestroy(stream));
    hipFree(x);
    hipFree(s);
    hipFree(g);
    if (b) hipFree(b);
    if (bias) hipFree(bias);
    hipFree(out);
    hipFree(out_ws);
    hipFree(out_static);
    if (res) hipFree(res);
    if (ws) hipFree(ws);
    free(h_x);
    free(h_s);
    free(h_g);
    free(h_b);
    free(h_bias);
    free(h_out);
    free(h_out_ws);
    free(h_out_static);
    return 0;
}
