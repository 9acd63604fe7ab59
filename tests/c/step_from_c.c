/* The hot path driven from plain C through the library's C ABI: device
 * buffers from hipMalloc, a stream from hipStreamCreate, then the calls a C
 * host program would make.
 *
 * step_from_c step <dir> <n> <w> <abar_t> <abar_prev>
 *   dfp_ddim_coeffs + dfp_cfg_step on one latent.
 *   reads  <dir>/x.f32, <dir>/g_c.f32, <dir>/g_u.f32   (n floats each)
 *   writes <dir>/x_out.f32 (n floats) and <dir>/relmae.f32 (1 float)
 * step_from_c attn <dir> <B> <H> <n_q> <N_kv> <d> <row0> <n>
 *   dfp_kv_scatter of the stale buffer, dfp_kv_scatter of the fresh patch
 *   rows at row0, dfp_patch_attention of the patch's queries (bf16, with a
 *   zeroed workspace so the key range may be split).
 *   reads  <dir>/q.bf16 [B,H,n_q,d], <dir>/k_stale.bf16, <dir>/v_stale.bf16
 *          [B,H,N_kv,d], <dir>/k_fresh.bf16, <dir>/v_fresh.bf16 [B,H,n,d]
 *   writes <dir>/o.bf16 [B,H,n_q,d]
 * Exit status 0 on success; a message on stderr otherwise. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dfp.h"

static int fail(const char *what, const char *detail) {
    fprintf(stderr, "step_from_c: %s: %s\n", what, detail);
    return 1;
}

static int read_raw(const char *dir, const char *name, void *dst, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return 0;
    const size_t got = fread(dst, 1, bytes, f);
    fclose(f);
    return got == bytes;
}

static int write_raw(const char *dir, const char *name, const void *src, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 0;
    const size_t put = fwrite(src, 1, bytes, f);
    fclose(f);
    return put == bytes;
}

#define read_f32(dir, name, dst, n) read_raw(dir, name, dst, sizeof(float) * (size_t)(n))
#define write_f32(dir, name, src, n) write_raw(dir, name, src, sizeof(float) * (size_t)(n))

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_));        \
    } while (0)

static int run_step(int argc, char **argv) {
    if (argc != 7) return fail("usage", "step_from_c step <dir> <n> <w> <abar_t> <abar_prev>");
    const char *dir = argv[2];
    const long n = atol(argv[3]);
    const float w = (float)atof(argv[4]);
    const double abar_t = atof(argv[5]), abar_prev = atof(argv[6]);
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

static int run_attn(int argc, char **argv) {
    if (argc != 10)
        return fail("usage", "step_from_c attn <dir> <B> <H> <n_q> <N_kv> <d> <row0> <n>");
    const char *dir = argv[2];
    const int B = atoi(argv[3]), H = atoi(argv[4]), n_q = atoi(argv[5]), N_kv = atoi(argv[6]);
    const int d = atoi(argv[7]), row0 = atoi(argv[8]), n = atoi(argv[9]);
    if (B <= 0 || H <= 0 || n_q <= 0 || N_kv <= 0 || d <= 0 || row0 < 0 || n <= 0 ||
        row0 + n > N_kv)
        return fail("sizes", "out of range");
    const size_t e = 2;   /* bf16 bit patterns */
    const size_t q_bytes = (size_t)B * H * n_q * d * e;
    const size_t kv_bytes = (size_t)B * H * N_kv * d * e;
    const size_t f_bytes = (size_t)B * H * n * d * e;
    const int64_t ldv = dfp_v_ld(N_kv, DFP_BF16);
    const size_t vt_bytes = (size_t)B * H * d * (size_t)ldv * e;
    unsigned char *h = malloc(q_bytes + 2 * kv_bytes + 2 * f_bytes);
    if (!h) return fail("malloc", "host buffers");
    unsigned char *hq = h, *hks = hq + q_bytes, *hvs = hks + kv_bytes, *hkf = hvs + kv_bytes;
    unsigned char *hvf = hkf + f_bytes;
    if (!read_raw(dir, "q.bf16", hq, q_bytes) || !read_raw(dir, "k_stale.bf16", hks, kv_bytes) ||
        !read_raw(dir, "v_stale.bf16", hvs, kv_bytes) ||
        !read_raw(dir, "k_fresh.bf16", hkf, f_bytes) ||
        !read_raw(dir, "v_fresh.bf16", hvf, f_bytes))
        return fail("read", "inputs");

    const size_t ws_bytes =
        dfp_workspace_bytes(DFP_OP_PATCH_ATTENTION, 0, 0, B, H, n_q, N_kv, d);
    void *dq = NULL, *do_ = NULL, *dkb = NULL, *dvt = NULL, *dks = NULL, *dvs = NULL;
    void *dkf = NULL, *dvf = NULL, *ws = NULL;
    hipStream_t stream = NULL;
    HIP_OK(hipStreamCreate(&stream));
    HIP_OK(hipMalloc(&dq, q_bytes));
    HIP_OK(hipMalloc(&do_, q_bytes));
    HIP_OK(hipMalloc(&dkb, kv_bytes));
    HIP_OK(hipMalloc(&dvt, vt_bytes));
    HIP_OK(hipMalloc(&dks, kv_bytes));
    HIP_OK(hipMalloc(&dvs, kv_bytes));
    HIP_OK(hipMalloc(&dkf, f_bytes));
    HIP_OK(hipMalloc(&dvf, f_bytes));
    if (ws_bytes) {
        HIP_OK(hipMalloc(&ws, ws_bytes));
        HIP_OK(hipMemsetAsync(ws, 0, ws_bytes, stream));   /* counters start at zero */
    }
    HIP_OK(hipMemcpyAsync(dq, hq, q_bytes, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(dks, hks, kv_bytes, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(dvs, hvs, kv_bytes, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(dkf, hkf, f_bytes, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(dvf, hvf, f_bytes, hipMemcpyHostToDevice, stream));

    dfp_status st = dfp_kv_scatter(dkb, dvt, dks, dvs, B, H, N_kv, d, 0, N_kv, DFP_BF16, stream);
    if (st != DFP_OK) return fail("dfp_kv_scatter (stale)", dfp_status_string(st));
    st = dfp_kv_scatter(dkb, dvt, dkf, dvf, B, H, N_kv, d, row0, n, DFP_BF16, stream);
    if (st != DFP_OK) return fail("dfp_kv_scatter (fresh)", dfp_status_string(st));
    st = dfp_patch_attention(do_, dq, dkb, dvt, B, H, n_q, N_kv, d, 1.0f / sqrtf((float)d),
                             DFP_BF16, ws, ws_bytes, stream);
    if (st != DFP_OK) return fail("dfp_patch_attention", dfp_status_string(st));

    HIP_OK(hipMemcpyAsync(hq, do_, q_bytes, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    if (!write_raw(dir, "o.bf16", hq, q_bytes)) return fail("write", "output");

    void *bufs[] = {dq, do_, dkb, dvt, dks, dvs, dkf, dvf, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    HIP_OK(hipStreamDestroy(stream));
    free(h);
    return 0;
}

int main(int argc, char **argv) {
    if (argc >= 2 && strcmp(argv[1], "step") == 0) return run_step(argc, argv);
    if (argc >= 2 && strcmp(argv[1], "attn") == 0) return run_attn(argc, argv);
    return fail("usage", "step_from_c step|attn ...");
}
