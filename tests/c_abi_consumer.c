/*
 * A plain C consumer of the library's C ABI (include/gemm.h, include/conv.h):
 * no Python, no torch.  It reads operands from raw little-endian files, moves
 * them to the GPU with the HIP runtime's C API, calls the library, and writes
 * the results back to files; tests/test_c_abi.py compares them with the
 * oracle.  It computes nothing itself.
 *
 * Usage: c_abi_consumer DIR
 *   DIR/shape.txt   "M N K"        then the 2-D convolution line
 *                   "batch cin h w cout r s pad"
 *   DIR/a_f32.bin, b_f32.bin       fp32 A (M x K) and B (K x N)
 *   DIR/a_bf16.bin, b_bf16.bin     bf16 bit patterns, same shapes
 *   DIR/at_bf16.bin, bt_bf16.bin   A^T (K x M) and B^T (N x K), bf16
 *   DIR/c0_bf16.bin                initial C (M x N), bf16
 *   DIR/x.bin, w.bin               fp32 image batch and filters
 * writes DIR/c_f32.out (gemm_f32), c_bf16.out (gemm_bf16), c_ex.out (gemm_ex:
 * bf16 C := 0.5 A^T.B^T - 2 C0), y.out (conv2d_fwd, fp32), and prints two
 * answers of the operand-copy query and the status string of one invalid
 * call.  Exit status 0 when every call
 * returned GEMM_OK (and the invalid one GEMM_ERR_INVALID_ARG).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "conv.h"
#include "gemm.h"

static void *read_file(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(2);
    }
    void *p = malloc(bytes ? bytes : 1);
    if (fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short read %s\n", path);
        exit(2);
    }
    fclose(f);
    return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(2);
    }
    fclose(f);
}

static void *to_device(const void *host, size_t bytes)
{
    void *d = NULL;
    if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess ||
        hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "device copy failed\n");
        exit(3);
    }
    return d;
}

static void *device_buffer(size_t bytes)
{
    void *d = NULL;
    if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess) {
        fprintf(stderr, "hipMalloc failed\n");
        exit(3);
    }
    return d;
}

static void to_host(void *host, const void *dev, size_t bytes)
{
    if (hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
        fprintf(stderr, "host copy failed\n");
        exit(3);
    }
}

static int check(const char *what, int rc, int want)
{
    if (rc != want) {
        fprintf(stderr, "%s: %s (%d)\n", what, gemm_status_string(rc), rc);
        return 1;
    }
    return 0;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 2;
    }
    const char *dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/shape.txt", dir);
    FILE *f = fopen(path, "r");
    long long M, N, K, nb, ci, h, w, co, r, s, pad;
    if (!f || fscanf(f, "%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", &M, &N, &K, &nb,
                     &ci, &h, &w, &co, &r, &s, &pad) != 11) {
        fprintf(stderr, "bad shape file\n");
        return 2;
    }
    fclose(f);
    const size_t mk = (size_t)(M * K), kn = (size_t)(K * N), mn = (size_t)(M * N);
    int bad = 0;

    /* plain products */
    float *a = read_file(dir, "a_f32.bin", mk * 4), *b = read_file(dir, "b_f32.bin", kn * 4);
    uint16_t *ah = read_file(dir, "a_bf16.bin", mk * 2), *bh = read_file(dir, "b_bf16.bin", kn * 2);
    float *dA = to_device(a, mk * 4), *dB = to_device(b, kn * 4), *dC = device_buffer(mn * 4);
    uint16_t *dAh = to_device(ah, mk * 2), *dBh = to_device(bh, kn * 2);
    float *c = malloc(mn * 4);
    bad |= check("gemm_f32", gemm_f32(M, N, K, dA, K, dB, N, dC, N, NULL), GEMM_OK);
    to_host(c, dC, mn * 4);
    write_file(dir, "c_f32.out", c, mn * 4);
    bad |= check("gemm_bf16", gemm_bf16(M, N, K, dAh, K, dBh, N, dC, N, NULL), GEMM_OK);
    to_host(c, dC, mn * 4);
    write_file(dir, "c_bf16.out", c, mn * 4);

    /* generalised: bf16 C := 0.5 A^T . B^T - 2 C0 */
    uint16_t *at = read_file(dir, "at_bf16.bin", mk * 2), *bt = read_file(dir, "bt_bf16.bin", kn * 2);
    uint16_t *c0 = read_file(dir, "c0_bf16.bin", mn * 2);
    uint16_t *dAt = to_device(at, mk * 2), *dBt = to_device(bt, kn * 2), *dC0 = to_device(c0, mn * 2);
    bad |= check("gemm_ex", gemm_ex(GEMM_DTYPE_BF16, GEMM_DTYPE_BF16, GEMM_OP_T, GEMM_OP_T, M, N, K,
                                    0.5f, dAt, M, dBt, K, -2.0f, dC0, N, NULL),
                 GEMM_OK);
    to_host(c0, dC0, mn * 2);
    write_file(dir, "c_ex.out", c0, mn * 2);

    /* 2-D convolution through im2col + GEMM, workspace from the size query */
    conv2d_params p = {nb, ci, h, w, co, r, s, pad, pad, 1, 1, 1, 1};
    int64_t P = 0, Q = 0;
    bad |= check("conv2d_output_size", conv2d_output_size(&p, &P, &Q), GEMM_OK);
    const size_t xs = (size_t)(nb * ci * h * w), ws_ = (size_t)(co * ci * r * s);
    const size_t ys = (size_t)(nb * co * P * Q);
    float *x = read_file(dir, "x.bin", xs * 4), *wt = read_file(dir, "w.bin", ws_ * 4);
    float *dx = to_device(x, xs * 4), *dw = to_device(wt, ws_ * 4), *dy = device_buffer(ys * 4);
    const int64_t need = conv2d_workspace_size(GEMM_DTYPE_F32, &p);
    if (need <= 0) {
        fprintf(stderr, "workspace query failed\n");
        return 1;
    }
    void *dws = device_buffer((size_t)need);
    bad |= check("conv2d_fwd", conv2d_fwd(GEMM_DTYPE_F32, GEMM_DTYPE_F32, &p, dx, dw, dy, dws, need,
                                          NULL),
                 GEMM_OK);
    float *y = malloc(ys * 4);
    to_host(y, dy, ys * 4);
    write_file(dir, "y.out", y, ys * 4);

    /* the operand-copy query (host only; the addresses are examined, not
       read): none for this call's aligned rows, both operands of an 8191^3
       bf16 product at odd pitches */
    printf("copy bytes: %lld %lld\n",
           (long long)gemm_operand_copy_bytes(GEMM_DTYPE_BF16, GEMM_OP_N, GEMM_OP_N, M, N, K, dAh, K,
                                              dBh, N),
           (long long)gemm_operand_copy_bytes(GEMM_DTYPE_BF16, GEMM_OP_N, GEMM_OP_N, 8191, 8191,
                                              8191, (const void *)(uintptr_t)0x100000, 8191,
                                              (const void *)(uintptr_t)0x100000, 8191));

    /* an invalid call: lda below the row length; nothing is launched */
    const int rc = gemm_f32(M, N, K, dA, K - 1, dB, N, dC, N, NULL);
    bad |= check("invalid lda", rc, GEMM_ERR_INVALID_ARG);
    printf("invalid call: %s\n", gemm_status_string(rc));

    if (hipDeviceSynchronize() != hipSuccess) {
        fprintf(stderr, "device error\n");
        return 3;
    }
    printf("%s\n", bad ? "FAILED" : "OK");
    return bad;
}
