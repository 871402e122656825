/*
 * A plain C client of libnormhip: no C++, no Python, no torch.  It checks
 * that include/normhip.h is valid C and that the library is usable through
 * its C ABI alone.
 *
 *   abi_client check
 *       Host-only: status strings, kernel names, the host self test, and
 *       argument validation of every entry point (no device needed).
 *   abi_client bn <in.bin> <out.bin>
 *       Reads N, C, HW (int64) and fp32 x[N*C*HW], dy[N*C*HW], gamma[C],
 *       beta[C]; runs bn_forward_train then bn_backward on the current HIP
 *       device with device buffers it allocates itself; writes fp32 y, stats
 *       [4*C], dx, grads [4*C].
 *   abi_client ln <in.bin> <out.bin>
 *       Reads rows, cols (int64) and fp32 x, dy [rows*cols], w [cols];
 *       runs layernorm_forward (mean, rstd) then layernorm_backward; writes
 *       fp32 y, mean, rstd, dx, dweight, dbias.
 * Exit status 0 on success; any failure prints the library's message.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "normhip.h"

#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); exit(1); } while (0)
#define NH(call) do { nh_status s_ = (call); \
    if (s_ != NH_OK) FAIL("%s -> %s: %s", #call, nh_status_string(s_), nh_last_error()); } while (0)
#define HIP(call) do { hipError_t e_ = (call); \
    if (e_ != hipSuccess) FAIL("%s -> %s", #call, hipGetErrorString(e_)); } while (0)
#define EXPECT(call, want) do { nh_status s_ = (call); \
    if (s_ != (want)) FAIL("%s -> %s, expected %s", #call, nh_status_string(s_), nh_status_string(want)); \
} while (0)

static void *fake = (void *)0x1000; /* never dereferenced: every call below fails first */

static int check(void)
{
    size_t ws = 0;
    if (strcmp(nh_status_string(NH_OK), "NH_OK") != 0) FAIL("status string");
    if (strcmp(nh_kernel_name(NH_K_BN_DX), "bn_dx") != 0) FAIL("kernel name");
    NH(nh_selftest_host());
    EXPECT(bn_forward_train(fake, fake, (nh_dtype)7, 2, 3, 4, NULL, NULL, NULL, NULL, 0.1f, 1e-5f,
                            fake, fake, 1u << 20, NULL), NH_ERR_DTYPE);
    EXPECT(bn_forward_train(NULL, fake, NH_F32, 2, 3, 4, NULL, NULL, NULL, NULL, 0.1f, 1e-5f,
                            fake, fake, 1u << 20, NULL), NH_ERR_NULL);
    EXPECT(bn_backward(fake, fake, NH_BF16, -1, 3, 4, fake, fake, fake, fake, 1u << 20, NULL),
           NH_ERR_SHAPE);
    EXPECT(bn_act_forward_train(fake, fake, NH_F32, 2, 3, 4, NULL, NULL, NULL, NULL, 0.1f, 1e-5f,
                                (nh_act)9, 0.f, fake, fake, 1u << 20, NULL), NH_ERR_ARG);
    EXPECT(bn_forward_infer(fake, fake, NH_F32, 2, 3, 4, NULL, NULL, NULL, fake, 1e-5f,
                            NH_ACT_RELU, 0.f, NULL), NH_ERR_NULL);
    EXPECT(layernorm_backward(fake, NH_BF16, fake, NH_F32, NULL, fake, NULL, NH_BF16, 4, 8, fake,
                              NH_F32, NULL, NULL, fake, 1u << 20, NULL), NH_ERR_NULL);
    EXPECT(rmsnorm_backward(fake, fake, (nh_dtype)2, NULL, 1e-5f, NULL, 4, 8, fake, NULL, fake,
                            1u << 20, NULL), NH_ERR_DTYPE);
    EXPECT(bda_layernorm_backward(fake, NH_BF16, fake, NH_F32, fake, fake, NULL, NH_BF16, NULL,
                                  NULL, 1.0f / 0.0f, 4, 8, NULL, NULL, NULL, NULL, NULL, fake,
                                  1u << 20, NULL), NH_ERR_ARG);
    EXPECT(layernorm_forward(fake, NH_F32, NULL, NULL, NH_F32, 4, 8, -1.f, fake, NH_F32, fake,
                             NULL, NULL), NH_ERR_ARG);
    EXPECT(rmsnorm_forward(NULL, NH_F32, NULL, 4, 8, 1e-5f, fake, NULL, NULL), NH_ERR_NULL);
    NH(bn_forward_train_workspace(0, 3, 4, &ws));
    if (ws != 0) FAIL("empty workspace");
    EXPECT(nh_plan_override("no_such_key", 1), NH_ERR_ARG);
    printf("check: ok\n");
    return 0;
}

static void *read_all(const char *path, size_t *n)
{
    FILE *f = fopen(path, "rb");
    if (!f) FAIL("cannot open %s", path);
    fseek(f, 0, SEEK_END);
    long len = ftell(f);
    fseek(f, 0, SEEK_SET);
    void *buf = malloc((size_t)len);
    if (!buf || fread(buf, 1, (size_t)len, f) != (size_t)len) FAIL("cannot read %s", path);
    fclose(f);
    *n = (size_t)len;
    return buf;
}

static void *to_device(const float *h, size_t count)
{
    void *d = NULL;
    HIP(hipMalloc(&d, count * sizeof(float) + 16));
    if (count) HIP(hipMemcpy(d, h, count * sizeof(float), hipMemcpyHostToDevice));
    return d;
}

static void append(FILE *f, const void *dev, size_t count)
{
    float *h = (float *)malloc(count * sizeof(float) + 1);
    HIP(hipMemcpy(h, dev, count * sizeof(float), hipMemcpyDeviceToHost));
    if (fwrite(h, sizeof(float), count, f) != count) FAIL("write failed");
    free(h);
}

static int run_bn(const char *in, const char *out)
{
    size_t n = 0;
    char *buf = (char *)read_all(in, &n);
    int64_t N, C, HW;
    memcpy(&N, buf, 8);
    memcpy(&C, buf + 8, 8);
    memcpy(&HW, buf + 16, 8);
    const size_t E = (size_t)(N * C * HW);
    if (n != 24 + 4 * (2 * E + 2 * (size_t)C)) FAIL("bn input size");
    const float *h = (const float *)(buf + 24);
    void *x = to_device(h, E), *dy = to_device(h + E, E);
    void *g = to_device(h + 2 * E, (size_t)C), *b = to_device(h + 2 * E + C, (size_t)C);
    void *y, *dx, *stats, *grads, *ws;
    size_t wsb = 0;
    NH(bn_forward_train_workspace(N, C, HW, &wsb));
    HIP(hipMalloc(&y, E * 4 + 16));
    HIP(hipMalloc(&dx, E * 4 + 16));
    HIP(hipMalloc(&stats, (size_t)C * 16));
    HIP(hipMalloc(&grads, (size_t)C * 16));
    HIP(hipMalloc(&ws, wsb + 16));
    NH(bn_forward_train(x, y, NH_F32, N, C, HW, (const float *)g, (const float *)b, NULL, NULL,
                        0.1f, 1e-5f, (float *)stats, ws, wsb, NULL));
    NH(bn_backward(dy, x, NH_F32, N, C, HW, (const float *)stats, dx, (float *)grads, ws, wsb,
                   NULL));
    HIP(hipDeviceSynchronize());
    FILE *f = fopen(out, "wb");
    if (!f) FAIL("cannot open %s", out);
    append(f, y, E);
    append(f, stats, 4 * (size_t)C);
    append(f, dx, E);
    append(f, grads, 4 * (size_t)C);
    fclose(f);
    hipFree(x); hipFree(dy); hipFree(g); hipFree(b); hipFree(y); hipFree(dx);
    hipFree(stats); hipFree(grads); hipFree(ws);
    free(buf);
    printf("bn: ok\n");
    return 0;
}

static int run_ln(const char *in, const char *out)
{
    size_t n = 0;
    char *buf = (char *)read_all(in, &n);
    int64_t R, H;
    memcpy(&R, buf, 8);
    memcpy(&H, buf + 8, 8);
    const size_t E = (size_t)(R * H);
    if (n != 16 + 4 * (2 * E + (size_t)H)) FAIL("ln input size");
    const float *h = (const float *)(buf + 16);
    void *x = to_device(h, E), *dy = to_device(h + E, E), *w = to_device(h + 2 * E, (size_t)H);
    void *y, *mean, *rstd, *dx, *dw, *db, *ws;
    size_t wsb = 0;
    NH(layernorm_backward_workspace(R, H, &wsb));
    HIP(hipMalloc(&y, E * 4 + 16));
    HIP(hipMalloc(&dx, E * 4 + 16));
    HIP(hipMalloc(&mean, (size_t)R * 4 + 16));
    HIP(hipMalloc(&rstd, (size_t)R * 4 + 16));
    HIP(hipMalloc(&dw, (size_t)H * 4 + 16));
    HIP(hipMalloc(&db, (size_t)H * 4 + 16));
    HIP(hipMalloc(&ws, wsb + 16));
    NH(layernorm_forward(x, NH_F32, w, NULL, NH_F32, R, H, 1e-5f, y, NH_F32, (float *)mean,
                         (float *)rstd, NULL));
    NH(layernorm_backward(dy, NH_F32, x, NH_F32, (const float *)mean, (const float *)rstd, w,
                          NH_F32, R, H, dx, NH_F32, dw, db, ws, wsb, NULL));
    HIP(hipDeviceSynchronize());
    FILE *f = fopen(out, "wb");
    if (!f) FAIL("cannot open %s", out);
    append(f, y, E);
    append(f, mean, (size_t)R);
    append(f, rstd, (size_t)R);
    append(f, dx, E);
    append(f, dw, (size_t)H);
    append(f, db, (size_t)H);
    fclose(f);
    hipFree(x); hipFree(dy); hipFree(w); hipFree(y); hipFree(dx); hipFree(mean); hipFree(rstd);
    hipFree(dw); hipFree(db); hipFree(ws);
    free(buf);
    printf("ln: ok\n");
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 2 && strcmp(argv[1], "check") == 0) return check();
    if (argc == 4 && strcmp(argv[1], "bn") == 0) return run_bn(argv[2], argv[3]);
    if (argc == 4 && strcmp(argv[1], "ln") == 0) return run_ln(argv[2], argv[3]);
    fprintf(stderr, "usage: %s check | bn <in> <out> | ln <in> <out>\n", argv[0]);
    return 2;
}
