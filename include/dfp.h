/*
 * dfp.h -- displaced patch attention and the fused guided sampler step on
 * AMD Instinct MI355X (gfx950).  C ABI of libdfp.so.
 *
 * The library computes one GPU's share of patch-parallel diffusion
 * inference:
 *   - the patch's fresh K/V land in a persistent full-image buffer whose
 *     other rows still hold the previous denoising step's K/V, and the patch's
 *     queries attend over that whole buffer;
 *   - once per step, the conditional and unconditional predictions are
 *     combined (classifier-free guidance), the latent is advanced by one
 *     DDIM (eta = 0) or flow-matching Euler step, and the rel-MAE between the
 *     two predictions is reduced;
 *   - a patch's GroupNorm takes its statistics from the other patches'
 *     previous-step partial sums and its own fresh ones (displaced GroupNorm,
 *     the corrected_async_gn mode).
 *
 * Sources (page title, section):
 *   [DF] "终极性能对比：DistriFusion vs 传统推理方案" -- "DistriFusion的革命性突破":
 *        early steps exchange activations synchronously; later steps reuse
 *        the previous step's activations and hide the exchange.
 *   [XD] "xDiT: an Inference Engine for Diffusion Transformers (DiTs) with
 *        Massive Parallelism" -- 三.2 PipeFusion (the image is cut into
 *        non-overlapping patches), 三.3 CFG Parallelism (cond and uncond
 *        behave as a batch of two; the two results are gathered before the
 *        scheduler runs).
 *   [HY] "Accelerating Diffusion via Hybrid Data-Pipeline Parallelism Based
 *        on Conditional Guidance Scheduling" -- 关键设计 2 (denoising
 *        discrepancy rel-MAE between the two predictions) and
 *        损失函数/训练策略 (flow matching uses the velocity v in place of eps).
 *   [AI] "AIGC 文生图系统如何优化扩散模型推理速度" -- section 3 (DDIM with
 *        eta; eta = 0 is deterministic) and section 6 (operator fusion to cut
 *        data movement).
 *   [DT] "DistriFusion高级教程：自定义并行配置实现超高清图像生成的完整指南" --
 *        多设备配置优化 and 速度与质量平衡: a communication mode named
 *        corrected_async_gn (an asynchronous GroupNorm with a correction),
 *        given by name only.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless the parameter says "host".  The
 *     caller owns every buffer; the library never allocates device memory.
 *   - Work is enqueued on `stream` and runs asynchronously; results are
 *     visible after the caller synchronises that stream.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns DFP_ERR_INVALID_ARG (or DFP_ERR_UNSUPPORTED for a
 *     shape/dtype the kernels do not implement) and touches no memory.
 *   - A launch error reported by the HIP runtime returns DFP_ERR_HIP.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - No entry point throws; none keeps state between calls except where a
 *     workspace is documented to (the attention split-KV arrival counters).
 *   - bf16 tensors hold raw bfloat16 bit patterns (uint16_t).
 *   - Tensors are dense and row-major in the order their shape is written,
 *     except the fresh K/V rows of dfp_kv_scatter_strided, which take
 *     element strides (so a projection's [B][N][H][d] output lands as is).
 *   - The persistent V buffer is stored TRANSPOSED ([B][H][d][ldv], see the
 *     layout block below), so the attention's P.V product reads it without a
 *     transpose; dfp_kv_scatter transposes fresh V rows once when they land,
 *     and dfp_patch_attention_fresh takes fresh V already channel-major.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef DFP_H
#define DFP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFP_OK = 0,
    DFP_ERR_INVALID_ARG = 1,  /* null pointer, negative or inconsistent size */
    DFP_ERR_UNSUPPORTED = 2,  /* valid request the kernels do not implement  */
    DFP_ERR_HIP = 3,          /* the HIP runtime rejected a launch           */
    DFP_ERR_TOO_LARGE = 4     /* exceeds the library's static scratch        */
} dfp_status;

typedef enum {
    DFP_F32 = 0,   /* float32                        */
    DFP_BF16 = 1   /* bfloat16 bit patterns (uint16) */
} dfp_dtype;

/* Operation ids for dfp_workspace_bytes. */
typedef enum {
    DFP_OP_CFG_STEP = 0,
    DFP_OP_RELMAE = 1,
    DFP_OP_PATCH_ATTENTION = 2
} dfp_op;

/* ------------------------------------------------------------------------
 * Persistent K/V buffer layout
 *
 * K buffer:  k_buf  [B][H][N_buf][d]      (one row per token)
 * V buffer:  v_buf_t[B][H][d][ldv]        (stored TRANSPOSED, one row per
 *                                          channel; ldv = dfp_v_ld(N_buf, dt))
 * ldv rounds N_buf up so every channel row starts on a 16-byte boundary;
 * columns N_buf..ldv-1 are padding that no kernel reads as data.  The
 * transposed V is what the attention kernel's P.V matrix product consumes
 * directly, so the transpose is paid once, when a patch lands, instead of in
 * every attention tile.
 * ------------------------------------------------------------------------ */

/* Row stride, in elements, of the transposed V buffer: N_buf rounded up to a
 * multiple of 8 (bf16) or 4 (f32).  Returns 0 for N_buf <= 0 or a bad dtype. */
int64_t dfp_v_ld(int64_t N_buf, dfp_dtype dt);

/* (a1) Land a patch's fresh K/V in the persistent buffer.
 * [DF]: after the warm-up steps a device attends over the previous step's
 * activations everywhere except its own patch; [XD] 三.2: a patch is one of
 * the image's non-overlapping token ranges, here rows [row0, row0+n).
 *
 *   k_buf   [B][H][N_buf][d]  in/out: rows row0..row0+n-1 of every (b,h)
 *                             are overwritten with k_new; others untouched.
 *   v_buf_t [B][H][d][ldv]    in/out: columns row0..row0+n-1 of every
 *                             channel row are overwritten with v_new
 *                             transposed; others untouched.
 *   k_new   [B][H][n][d]      this step's keys of the patch.
 *   v_new   [B][H][n][d]      this step's values of the patch.
 * Bit-exact copy, no arithmetic.  Either k pair or v pair may be NULL (both
 * of a pair) to land only the other.  n == 0 is a no-op (pointers may then
 * be NULL).
 * d must be a multiple of 8 (bf16) or 4 (f32).
 * Errors: INVALID_ARG for row0 < 0, row0 + n > N_buf, non-positive B/H/d/N_buf,
 * negative n, or a half-null pair; UNSUPPORTED for other d or dtype. */
dfp_status dfp_kv_scatter(void *k_buf, void *v_buf_t, const void *k_new,
                          const void *v_new, int B, int H, int N_buf, int d,
                          int row0, int n, dfp_dtype dt, hipStream_t stream);

/* dfp_kv_scatter for fresh rows in any layout whose rows are contiguous: row
 * i of (b, h) starts at element b * stride_b + h * stride_h + i * stride_n of
 * k_new (and of v_new, which shares the strides), and holds d contiguous
 * elements.  A projection's [B][n][H][d] output passes stride_b = n*H*d,
 * stride_h = d, stride_n = H*d; dense [B][H][n][d] is stride_b = H*n*d,
 * stride_h = n*d, stride_n = d (what dfp_kv_scatter passes).  Strides are in
 * elements, non-negative, multiples of 8 (bf16) or 4 (f32) so every row
 * starts on a 16-byte boundary, and stride_n >= d; the caller guarantees
 * every addressed row lies inside its tensors.  Result, buffers, other
 * arguments and errors as dfp_kv_scatter, plus INVALID_ARG for a stride
 * outside these rules. */
dfp_status dfp_kv_scatter_strided(void *k_buf, void *v_buf_t, const void *k_new,
                                  const void *v_new, int B, int H, int N_buf, int d,
                                  int row0, int n, int64_t stride_b, int64_t stride_h,
                                  int64_t stride_n, dfp_dtype dt, hipStream_t stream);

/* (a2-a4) One patch's attention over the displaced buffer.
 * [DF] activation reuse: the buffer holds fresh rows for this patch (and
 * any always-fresh rows such as a DiT's text tokens) and the previous step's
 * rows elsewhere; the attention itself is plain softmax attention over all
 * N_kv buffer rows:
 *   O[b,h,i,:] = sum_j softmax_j(scale * <Q[b,h,i,:], K[b,h,j,:]>) V[b,h,j,:]
 * with no mask, bias or dropout.
 *
 *   o       [B][H][n_q][d]    output, dtype dt (fp32 accumulation inside).
 *   q       [B][H][n_q][d]    the patch's queries, dtype dt.
 *   k_buf   [B][H][N_kv][d]   dtype dt.
 *   v_buf_t [B][H][d][ldv]    dtype dt, ldv = dfp_v_ld(N_kv, dt).
 *   scale   softmax scale, normally 1/sqrt(d); must be finite and > 0.
 *   workspace/ws_bytes  optional device scratch (may be NULL/0), 256-byte
 *           aligned.  With at least dfp_workspace_bytes(DFP_OP_PATCH_ATTENTION,
 *           ...) bytes the kernel may split the key range across workgroups
 *           when the query grid alone is too small to fill the GPU; without
 *           it, it never splits.  The workspace starts with per-query-tile
 *           arrival counters that must be zero before the first call (e.g.
 *           allocate it zeroed); every call leaves them zero again.  How
 *           many counters there are, and so where the partials begin,
 *           depends on the sizes and the plan: zero the workspace again
 *           before it serves calls of other sizes, or keep one per size.
 *           The split partials are merged in a fixed order, so results are
 *           bitwise reproducible for a given shape.  Calls that share a
 *           workspace must not run concurrently (one stream, or streams
 *           ordered by events).
 * d must be 64 or 128.  n_q == 0 is a no-op (pointers may then be NULL).
 * o must not alias the inputs.
 * Errors: INVALID_ARG for null pointers, non-positive B/H/N_kv, negative n_q,
 * a bad scale, pointers not 16-byte aligned; UNSUPPORTED for other d or
 * dtype, or (bf16) when one (b,h) slice of k_buf or v_buf_t reaches 2 GiB. */
dfp_status dfp_patch_attention(void *o, const void *q, const void *k_buf,
                               const void *v_buf_t, int B, int H, int n_q,
                               int N_kv, int d, float scale, dfp_dtype dt,
                               void *workspace, size_t ws_bytes,
                               hipStream_t stream);

/* One range of fresh rows for dfp_patch_attention_fresh: this step's keys
 * and values of buffer rows row0..row0+n-1.
 *   k    [B][H][n][d]   device pointer, 16-byte aligned.
 *   v_t  [B][H][d][n]   device pointer, 16-byte aligned; values stored
 *                       TRANSPOSED (channel-major), as the buffer stores V --
 *                       a projection can emit this layout directly by
 *                       swapping its GEMM operands.
 *   row0, n             multiples of 64 (whole 64-key tiles). */
typedef struct {
    const void *k;
    const void *v_t;
    int row0;
    int n;
} dfp_fresh_rows;

/* (a1-a4) One patch's attention with its fresh rows read straight from this
 * step's K/V, and (optionally) their landing in the buffer, in one launch.
 * [DF]: the device computes fresh activations for its own patch (and a
 * DiT's always-fresh text tokens) and attends over them together with the
 * previous step's activations of every other patch; the fresh ones are also
 * what the next step reuses.  The result is dfp_patch_attention over the
 * buffer with the rows of every fresh range replaced by that range's rows;
 * the buffer's own rows there are never read, so the landing (land != 0)
 * can write them during the same launch, exactly as dfp_kv_scatter(k,
 * transpose(v_t), row0) of each range would.
 *
 *   o, q, scale, workspace/ws_bytes   as dfp_patch_attention (bf16 only).
 *   k_buf   [B][H][N_kv][d]   read outside the fresh ranges; rows inside are
 *                             overwritten with the fresh keys when land != 0.
 *   v_buf_t [B][H][d][ldv]    likewise for the fresh columns.
 *   fresh   host array of n_fresh (1 or 2) non-overlapping ranges.
 * Inputs must not alias the buffer.  With land == 0 the buffer is not
 * written.  n_q == 0 with land != 0 only lands (o and q may then be NULL).
 * Errors: INVALID_ARG for null or misaligned pointers, a NULL fresh array or
 * n_fresh < 1, a range with n <= 0, row0 < 0 or row0 + n > N_kv, overlapping
 * ranges, non-positive B/H/N_kv, negative n_q, a bad scale; UNSUPPORTED for
 * n_fresh > 2, dt other than bf16, d other than 64/128, a range not made of
 * whole 64-key tiles, or a (b,h) slice of k_buf or v_buf_t reaching 2 GiB. */
dfp_status dfp_patch_attention_fresh(void *o, const void *q, void *k_buf,
                                     void *v_buf_t, const dfp_fresh_rows *fresh,
                                     int n_fresh, int B, int H, int n_q, int N_kv,
                                     int d, int land, float scale, dfp_dtype dt,
                                     void *workspace, size_t ws_bytes,
                                     hipStream_t stream);

/* (a5-a7) Fused guidance + sampler update + rel-MAE, one pass over HBM.
 * [XD] 三.3 / [HY] 关键设计 1: the step consumes a conditional and an
 * unconditional prediction of the same latent.  Per element (fp32):
 *   g  = g_u + w * (g_c - g_u)              classifier-free guidance
 *   x <- c_x * x + c_e * g                  sampler update, in place
 * and per image b (batch index), before guidance is applied:
 *   relmae_out[b] = sum |g_c - g_u| / sum |g_u|        ([HY] 关键设计 2)
 * The affine form covers DDIM eta = 0 ([AI] section 3; see dfp_ddim_coeffs)
 * and Euler on sigma (see dfp_euler_coeffs).
 *
 *   x          [batch][n_per_image] fp32, updated in place.
 *   g_c, g_u   [batch][n_per_image] fp32.
 *   relmae_out [batch] fp32 device memory, or NULL to skip the reduction.
 *   workspace  device scratch of >= dfp_workspace_bytes(DFP_OP_CFG_STEP,
 *              n_per_image, batch, ...) bytes, 16-byte aligned, required when
 *              relmae_out is non-NULL; its initial contents do not matter.
 *              It receives one fp64 (sum, sum) pair per workgroup, which a
 *              second launch of the call (one wavefront per image) sums in
 *              a fixed order in double precision, so results are bitwise
 *              reproducible for a given size and entry point.  Calls that share a workspace
 *              must not run concurrently.
 * Degenerate rel-MAE follows IEEE division (0/0 = NaN, x/0 = +Inf).
 * Errors: INVALID_ARG for null x/g_c/g_u, n_per_image <= 0, batch <= 0,
 * a missing or short workspace when relmae_out is non-NULL, non-finite
 * w/c_x/c_e. */
dfp_status dfp_cfg_step(float *x, const float *g_c, const float *g_u,
                        int64_t n_per_image, int batch, float w, double c_x,
                        double c_e, float *relmae_out, void *workspace,
                        size_t ws_bytes, hipStream_t stream);

/* Fused step with a noise term: DDIM with eta > 0 ([AI] section 3, the
 * sigma_eta * z term of the same update).  Per element:
 *   x <- c_x * x + c_e * g + c_z * z
 * with g the guided prediction as above and z a standard-normal draw the
 * caller supplies (same shape and layout as x; drawn by the caller so any
 * generator can feed the step).  See dfp_ddim_eta_coeffs for (c_x, c_e, c_z).
 * rel-MAE, workspace rules and errors are those of dfp_cfg_step, plus
 * INVALID_ARG for a null z or non-finite c_z.  Reads 20 bytes and writes 4
 * per element. */
dfp_status dfp_cfg_step_noise(float *x, const float *g_c, const float *g_u,
                              const float *z, int64_t n_per_image, int batch,
                              float w, double c_x, double c_e, double c_z,
                              float *relmae_out, void *workspace,
                              size_t ws_bytes, hipStream_t stream);

/* Fused step with the noise term drawn inside the kernel: DDIM with eta > 0
 * ([AI] section 3, the sigma_eta * z term with z drawn by randn_like) at the
 * 16 bytes per element of dfp_cfg_step.  Per element:
 *   x <- c_x * x + c_e * g + c_z * z
 * with z the standard-normal draw of this image and step from a counter-based
 * generator, so any device (or the host) draws the same z:
 *   elements 8j .. 8j+7 of image b (b = batch index of this call) come from
 *   the Philox4x64-10 block (J. Salmon et al., "Parallel Random Numbers: As
 *   Easy as 1, 2, 3", SC'11) of counter (j, b, 0, 0) under key (seed, step);
 *   its four 64-bit words' 32-bit halves h_0..h_7 (h_2k the low half of word
 *   k) become u_m = (h_m + 1/2) / 2^32, and Box-Muller gives
 *     z[8j+2k]   = sqrt(-2 ln u_2k) cos(2 pi u_2k+1)
 *     z[8j+2k+1] = sqrt(-2 ln u_2k) sin(2 pi u_2k+1).
 * The device evaluates the transform in fp32 (|z - z_exact| stays within a
 * few fp32 ulps of |z|).  seed, step: any 64-bit values; a sampler passes
 * its seed and the step index.  rel-MAE, workspace rules and errors are
 * those of dfp_cfg_step, plus INVALID_ARG for a non-finite c_z.  Reads 12
 * bytes and writes 4 per element. */
dfp_status dfp_cfg_step_philox(float *x, const float *g_c, const float *g_u,
                               int64_t n_per_image, int batch, float w, double c_x,
                               double c_e, double c_z, uint64_t seed, uint64_t step,
                               float *relmae_out, void *workspace, size_t ws_bytes,
                               hipStream_t stream);

/* The draw z that dfp_cfg_step_philox adds, written out (same device code):
 *   z  [batch][n_per_image] fp32 device output.
 * Errors: INVALID_ARG for a null z, n_per_image <= 0, batch outside
 * [1, 65535]. */
dfp_status dfp_philox_normal(float *z, int64_t n_per_image, int batch, uint64_t seed,
                             uint64_t step, hipStream_t stream);

/* Raw Philox4x64-10 blocks (the generator under dfp_cfg_step_philox):
 *   out [blocks][4] uint64 device output; block j is the generator applied to
 *   counter (j, counter1, 0, 0) under key (key0, key1).
 * blocks == 0 is a no-op.  Errors: INVALID_ARG for blocks < 0 or a null out. */
dfp_status dfp_philox4x64_10(uint64_t *out, int64_t blocks, uint64_t counter1, uint64_t key0,
                             uint64_t key1, hipStream_t stream);

/* dfp_cfg_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as dfp_cfg_step without the workspace: the
 * rel-MAE partials go to a static device array of
 * dfp_cfg_static_scratch_bytes() bytes (1 MiB) inside the library, one per
 * GPU, kept until the process ends.  Nothing in it needs initial contents.
 * The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks the array's device address up
 * once.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams without ordering, several host
 * threads) race and may return wrong rel-MAE values.
 * Errors: those of dfp_cfg_step, and DFP_ERR_TOO_LARGE (nothing enqueued)
 * when relmae_out is non-NULL and dfp_workspace_bytes(DFP_OP_CFG_STEP,
 * n_per_image, batch, ...) exceeds dfp_cfg_static_scratch_bytes(). */
dfp_status dfp_cfg_step_static(float *x, const float *g_c, const float *g_u,
                               int64_t n_per_image, int batch, float w, double c_x,
                               double c_e, float *relmae_out, hipStream_t stream);

/* Size in bytes of the static scratch of dfp_cfg_step_static. */
size_t dfp_cfg_static_scratch_bytes(void);

/* (a7) rel-MAE alone ([HY] 关键设计 2):
 *   out[b] = sum |g_c - g_u| / sum |g_u|  over image b's n_per_image values.
 * Same reduction, workspace rules and errors as dfp_cfg_step. */
dfp_status dfp_relmae(const float *g_c, const float *g_u, int64_t n_per_image,
                      int batch, float *out, void *workspace, size_t ws_bytes,
                      hipStream_t stream);

/* (f4) Displaced GroupNorm of one patch: the corrected_async_gn mode that
 * [DT] 多设备配置优化 names (an asynchronous GroupNorm with a correction;
 * the page gives only the name).  Reading, after [DF] 革命性突破's reuse of
 * the previous step's activations: each group's statistics sum every other
 * patch's partial sums from the previous step (stale) and this patch's own
 * sums from this step (fresh, the correction); all P patches have n
 * positions.  Per image b and group g (channels g*C/G .. (g+1)*C/G - 1):
 *   f1 = sum x, f2 = sum x^2 over the patch's group   (fp64)
 *   S1 = f1 + sum_{q != p} stats[b][g][q][0],  S2 likewise with [1]
 *   N = P * n * C/G,  mean = S1/N,  var = S2/N - mean^2 (biased)
 *   y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c]
 *
 *   y      [B][C][n]     fp32 output; may equal x (in place), must not
 *                        otherwise overlap it.
 *   x      [B][C][n]     fp32, this patch's activations (NCHW with the
 *                        patch's rows contiguous: n = rows * width).
 *   stats  [B][G][P][2]  fp64 device buffer, 8-byte aligned: each patch's
 *                        (sum, sum of squares) of the previous step.  Slot
 *                        p is ignored on input; with land != 0 it receives
 *                        (f1, f2) for the next step.
 *   gamma, beta  [C] fp32, or NULL (1 and 0).
 *   workspace/ws_bytes  optional device scratch (may be NULL/0), 8-byte
 *           aligned; its initial contents do not matter.  A patch's group
 *           of up to 64 Ki floats (C/G * n, with n % 4 == 0 and x, y 16-byte
 *           aligned) needs none: one workgroup per (image, group) holds it
 *           in registers (one read of x).  Longer groups, with at least
 *           dfp_group_norm_workspace_bytes(B, C, G, n) bytes, are cut into
 *           chunks of 4 Ki floats spread over the whole GPU in two launches
 *           (chunk sums, then statistics and normalization; x is read
 *           twice); without it one workgroup per (image, group) streams x
 *           twice.  Calls that share a workspace must not run
 *           concurrently.
 * The statistics are bitwise reproducible (fixed-order fp64 sums).
 * Errors: INVALID_ARG for null y/x/stats, non-positive B/C/G/n/P, C not a
 * multiple of G, p outside [0, P), negative or non-finite eps, misaligned
 * stats, y partially overlapping x; UNSUPPORTED for B > 65535. */
dfp_status dfp_displaced_group_norm(float *y, const float *x, double *stats,
                                    const float *gamma, const float *beta, int B,
                                    int C, int G, int64_t n, int P, int p,
                                    float eps, int land, void *workspace,
                                    size_t ws_bytes, hipStream_t stream);

/* Workspace bytes dfp_displaced_group_norm uses for these sizes to spread
 * long groups over the GPU (0: none needed, or invalid sizes). */
size_t dfp_group_norm_workspace_bytes(int B, int C, int G, int64_t n);

/* Device scratch, in bytes, that `op` needs for the given sizes.  Arguments
 * that do not apply to `op` are ignored.  Returns 0 if the op needs none. */
size_t dfp_workspace_bytes(int op, int64_t n_per_image, int batch, int B, int H,
                           int n_q, int N_kv, int d);

/* How a bf16 dfp_patch_attention or dfp_patch_attention_fresh call of these
 * sizes is laid out on the GPU (host-only query, no GPU work).  The launch
 * depends only on the sizes, on whether a big enough workspace is passed
 * (with_workspace != 0) and on the environment overrides DFP_ATTN_SPLITS and
 * DFP_ATTN_KS read at each call.  Outputs (HOST pointers, each may be NULL):
 *   key_groups  1, or 2 when every workgroup splits its key range between
 *               two groups of wavefronts and merges them on chip (d = 64,
 *               grids too small to fill the GPU);
 *   splits      workgroups sharing one query tile's key range (> 1 only
 *               with a workspace);
 *   workgroups  attention workgroups of the launch (a fresh call adds its
 *               landing workgroups).
 * Errors: INVALID_ARG for non-positive B/H/n_q/N_kv; UNSUPPORTED for d other
 * than 64/128 or B*H beyond int range. */
dfp_status dfp_attention_plan(int B, int H, int n_q, int N_kv, int d,
                              int with_workspace, int *key_groups, int *splits,
                              int64_t *workgroups);

/* ------------------------------------------------------------------------
 * Host helpers (no GPU work).  All outputs are HOST pointers.
 * ------------------------------------------------------------------------ */

/* [AI] section 3 DDIM, eta = 0, folded to x' = c_x x + c_e g:
 *   c_x = sqrt(abar_prev / abar_t)
 *   c_e = sqrt(1 - abar_prev) - sqrt(abar_prev) sqrt(1 - abar_t) / sqrt(abar_t)
 * Pass abar_prev = 1 on the last step (the step that returns the x0 estimate).
 * INVALID_ARG unless 0 < abar_t <= 1 and 0 < abar_prev <= 1, or a null output. */
dfp_status dfp_ddim_coeffs(double abar_t, double abar_prev, double *c_x, double *c_e);

/* [AI] section 3 DDIM with noise scale eta, folded to
 * x' = c_x x + c_e g + c_z z:
 *   sigma = eta sqrt((1 - abar_prev)/(1 - abar_t) (1 - abar_t/abar_prev))
 *   c_x = sqrt(abar_prev / abar_t)
 *   c_e = sqrt(1 - abar_prev - sigma^2) - sqrt(abar_prev) sqrt(1 - abar_t) / sqrt(abar_t)
 *   c_z = sigma
 * eta = 0 gives dfp_ddim_coeffs with c_z = 0; abar_prev = 1 (last step) gives
 * c_z = 0 for any eta.  INVALID_ARG unless 0 < abar_t < 1, abar_t <= abar_prev
 * <= 1, eta >= 0 finite and 1 - abar_prev - sigma^2 >= 0 (always so for
 * eta <= 1), or for a null output. */
dfp_status dfp_ddim_eta_coeffs(double abar_t, double abar_prev, double eta, double *c_x,
                               double *c_e, double *c_z);

/* Euler on sigma: x' = x + (sigma_next - sigma) v, i.e. c_x = 1,
 * c_e = sigma_next - sigma.  INVALID_ARG for non-finite input or null output. */
dfp_status dfp_euler_coeffs(double sigma, double sigma_next, double *c_x, double *c_e);

/* Three-phase switch points from a rel-MAE series ("Accelerating Diffusion via
 * Hybrid Data-Pipeline Parallelism Based on Conditional Guidance Scheduling",
 * 关键设计 3).  relmae: host, S values, relmae[t] the discrepancy of step t
 * (t = 0 the first, noisiest step), e.g. the per-step outputs of
 * dfp_cfg_step.  With G_t = (relmae[t] - relmae[t-L]) / L for t >= L:
 *   tau1' = first t with 0 <= G_t < g_slope,
 *   tau_cap = first step of the series' minimum,
 *   tau1 = min(tau1', tau_cap) (tau_cap if there is no such t),
 *   tau2 = min(tau1 + k, S).
 * Warm-up is steps [0, tau1], parallel (tau1, tau2), fully-connecting
 * [tau2, S).  The page fixes k = 5 and leaves L and g_slope open; tau_cap
 * needs the whole series (e.g. from a profiling run).
 * INVALID_ARG for null pointers, S < 1, L < 1, k < 0, non-finite g_slope or
 * a non-finite series value. */
dfp_status dfp_switch_points(const float *relmae, int S, int L, double g_slope, int k,
                             int *tau1, int *tau2);

/* The scaled-linear schedule: beta_i = (sqrt(b0) + (sqrt(b1)-sqrt(b0)) i/(T-1))^2,
 * abar[t] = prod_{i<=t} (1 - beta_i), t = 0..T-1.  abar: host, T doubles. */
dfp_status dfp_scaled_linear_abar(int T, double beta_start, double beta_end, double *abar);

/* DDIM timesteps: round-half-even of linspace(0, T-1, S), ascending.
 * ts: host, S ints.  The sampler walks them in reverse ([AI] section 3). */
dfp_status dfp_ddim_timesteps(int T, int S, int *ts);

/* Static text for a status code. */
const char *dfp_status_string(dfp_status s);

#ifdef __cplusplus
}
#endif

#endif /* DFP_H */
