/* One fused guidance step driven from plain C through the library's C ABI:
 * device buffers from hipMalloc, a stream from hipStreamCreate, then
 * dfp_ddim_coeffs and dfp_cfg_step, as a C host program would call them.
 *
 * usage: step_from_c <dir> <n> <w> <abar_t> <abar_prev>
 * reads  <dir>/x.f32, <dir>/g_c.f32, <dir>/g_u.f32   (n floats each)
 * writes <dir>/x_out.f32 (n floats) and <dir>/relmae.f32 (1 float)
 * Exit status 0 on success; a message on stderr otherwise. */
#include <stdio.h>
#include <stdlib.h>

#include "dfp.h"

static int fail(const char *what, const char *detail) {
    fprintf(stderr, "step_from_c: %s: %s\n", what, detail);
    return 1;
}

static int read_f32(const char *dir, const char *name, float *dst, long n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return 0;
    const size_t got = fread(dst, sizeof(float), (size_t)n, f);
    fclose(f);
    return got == (size_t)n;
}

static int write_f32(const char *dir, const char *name, const float *src, long n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 0;
    const size_t put = fwrite(src, sizeof(float), (size_t)n, f);
    fclose(f);
    return put == (size_t)n;
}

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_));        \
    } while (0)

int main(int argc, char **argv) {
    if (argc != 6) return fail("usage", "step_from_c <dir> <n> <w> <abar_t> <abar_prev>");
    const char *dir = argv[1];
    const long n = atol(argv[2]);
    const float w = (float)atof(argv[3]);
    const double abar_t = atof(argv[4]), abar_prev = atof(argv[5]);
    if (n <= 0) return fail("n", "must be positive");

    float *h = malloc(sizeof(float) * (size_t)n * 3);
    if (!h) return fail("malloc", "host buffers");
    float *hx = h, *hc = h + n, *hu = h + 2 * n;
    if (!read_f32(dir, "x.f32", hx, n) || !read_f32(dir, "g_c.f32", hc, n) ||
        !read_f32(dir, "g_u.f32", hu, n))
        return fail("read", "inputs");

    double c_x = 0.0, c_e = 0.0;
    dfp_status st = dfp_ddim_coeffs(abar_t, abar_prev, &c_x, &c_e);
    if (st != DFP_OK) return fail("dfp_ddim_coeffs", dfp_status_string(st));

    const size_t ws_bytes = dfp_workspace_bytes(DFP_OP_CFG_STEP, n, 1, 0, 0, 0, 0, 0);
    float *dx = NULL, *dc = NULL, *du = NULL, *dr = NULL;
    void *ws = NULL;
    hipStream_t stream = NULL;
    HIP_OK(hipStreamCreate(&stream));
    HIP_OK(hipMalloc((void **)&dx, sizeof(float) * (size_t)n));
    HIP_OK(hipMalloc((void **)&dc, sizeof(float) * (size_t)n));
    HIP_OK(hipMalloc((void **)&du, sizeof(float) * (size_t)n));
    HIP_OK(hipMalloc((void **)&dr, sizeof(float)));
    HIP_OK(hipMalloc(&ws, ws_bytes));
    HIP_OK(hipMemcpyAsync(dx, hx, sizeof(float) * (size_t)n, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(dc, hc, sizeof(float) * (size_t)n, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(du, hu, sizeof(float) * (size_t)n, hipMemcpyHostToDevice, stream));

    st = dfp_cfg_step(dx, dc, du, n, 1, w, c_x, c_e, dr, ws, ws_bytes, stream);
    if (st != DFP_OK) return fail("dfp_cfg_step", dfp_status_string(st));

    float r = 0.f;
    HIP_OK(hipMemcpyAsync(hx, dx, sizeof(float) * (size_t)n, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(&r, dr, sizeof(float), hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    if (!write_f32(dir, "x_out.f32", hx, n) || !write_f32(dir, "relmae.f32", &r, 1))
        return fail("write", "outputs");

    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(dr));
    HIP_OK(hipFree(du));
    HIP_OK(hipFree(dc));
    HIP_OK(hipFree(dx));
    HIP_OK(hipStreamDestroy(stream));
    free(h);
    return 0;
}
