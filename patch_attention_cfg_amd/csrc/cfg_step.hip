// cfg_step.hip -- one fused, bandwidth-bound pass per denoising step:
// classifier-free guidance, the affine sampler update of the latent (with
// an optional sampler-noise term), and the rel-MAE reduction between the two
// predictions.
//
// Sources (page title, section):
//   "xDiT: an Inference Engine for Diffusion Transformers (DiTs) with Massive
//   Parallelism", 三.3 CFG Parallelism: the conditional and unconditional
//   predictions are gathered before the scheduler step.
//   "Accelerating Diffusion via Hybrid Data-Pipeline Parallelism Based on
//   Conditional Guidance Scheduling", 关键设计 2: rel-MAE of the two noise
//   predictions, taken as sum|g_c - g_u| / sum|g_u| over one image; and
//   损失函数/训练策略: flow-matching models use the velocity instead of eps.
//   "AIGC 文生图系统如何优化扩散模型推理速度", section 3 (DDIM; with eta > 0
//   the step adds sigma * z for a standard-normal z) and section 6 (operator
//   fusion cuts data movement): guidance, update and reduction share one read
//   of g_c and g_u, so the step moves 16 bytes per latent element (x read +
//   write, g_c and g_u read) -- also with eta > 0 when z is drawn in the
//   kernel from a counter-based generator instead of read from memory.
//
// Launch shape: one image's elements are spread over as many workgroups as
// it takes for every thread to hold one pass of loads (up to kMaxBlocks per
// image, grid-stride beyond), so a whole SDXL-3840 latent is in flight at
// once across the GPU.
//
// Reduction: fp32 per thread and per wavefront, fp64 per workgroup, stored
// to the workspace; a second, one-workgroup-per-image launch sums each
// image's partials in a fixed order in fp64 and writes the ratio.  No float
// atomics and no arrival counters, so the result is bitwise reproducible and
// the workspace needs no initial contents.  (Measured on MI355X for one
// SDXL-3840 latent: the data pass alone takes 3.4 us; a last-arriving
// workgroup merging in the same launch costs a chain of memory round trips
// -- publish, arrive, read back -- and, with every workgroup arriving on
// one counter, about 14 ns per workgroup of serialized atomics; the
// following launch is cheaper than either.)
#include <cmath>
#include <mutex>

#include "dfp_common.h"
#include "dfp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / dfp::kWave;
constexpr int kUnroll = 2;        // items per thread per pass, kThreads apart
constexpr int kMaxBlocks = 4096;  // workgroups per image, at most

// Items per thread per pass: one with drawn noise (8 floats and a Philox
// block each, so the generator's arithmetic spreads over twice the
// wavefronts), kUnroll otherwise.
template <int NOISE>
constexpr int unroll_of() { return NOISE == 2 ? 1 : kUnroll; }

// Workgroups per image for items of `item_floats` floats, `unroll` per
// thread and pass.  Items of 8 floats at one per thread give the same count
// as items of 4 at kUnroll = 2, so the workspace (sized for the latter)
// always fits.
inline int plan_blocks(int64_t n_per_image, int item_floats, int unroll = kUnroll) {
    const int64_t items = (n_per_image + item_floats - 1) / item_floats;
    const int64_t per_wg = (int64_t)kThreads * unroll;
    int64_t b = (items + per_wg - 1) / per_wg;
    if (b > kMaxBlocks) b = kMaxBlocks;
    return (int)(b < 1 ? 1 : b);
}

// --------------------------------------------------------- sampler noise
// The standard-normal draw z of a DDIM step with eta > 0, from Philox4x64
// with 10 rounds (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11) and the Box-Muller transform.
// Elements 8j .. 8j+7 of image b come from the block of counter (j, b, 0, 0)
// under key (seed, step): its words' 32-bit halves h (low half of word k
// first) become uniforms u = (h + 1/2) 2^-32, and pair k gives
//   z[8j+2k] = sqrt(-2 ln u_2k) cos(2 pi u_2k+1),
//   z[8j+2k+1] = sqrt(-2 ln u_2k) sin(2 pi u_2k+1).

// Full 128-bit product of two 64-bit words from four 32 x 32 -> 64 products.
__device__ __forceinline__ void mul128(uint64_t a, uint64_t b, uint64_t &lo, uint64_t &hi) {
    const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
    const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
    const uint64_t p00 = (uint64_t)a0 * b0, p01 = (uint64_t)a0 * b1;
    const uint64_t p10 = (uint64_t)a1 * b0, p11 = (uint64_t)a1 * b1;
    const uint64_t mid = (p00 >> 32) + (uint32_t)p01 + (uint32_t)p10;   // < 3 * 2^32
    lo = (mid << 32) | (uint32_t)p00;
    hi = p11 + (p01 >> 32) + (p10 >> 32) + (mid >> 32);
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t lo0, hi0, lo1, hi1;
        mul128(M0, c[0], lo0, hi0);
        mul128(M1, c[2], lo1, hi1);
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// ln u for u = (h + 1/2) 2^-32 in fp32 on the hardware log2: directly
// where u <= 1 - 2^-7, and from the exact complement y = 1 - u through the
// series ln(1 - y) = -y (1 + y/2 + y^2/3 + y^3/4 + ...) above it, where
// forming u itself in fp32 would lose y's low bits (the dropped terms are
// below 2^-30 relative there).
__device__ __forceinline__ float ln_uniform(uint32_t h) {
    const float u = fmaf((float)h, 0x1p-32f, 0x1p-33f);
    const float y = fmaf((float)(0xFFFFFFFFu - h), 0x1p-32f, 0x1p-33f);
    const float direct = __builtin_amdgcn_logf(u) * 0.69314718055994531f;
    const float series = -y * fmaf(y, fmaf(y, fmaf(y, 0.25f, 0.33333333f), 0.5f), 1.0f);
    return y < 0x1p-7f ? series : direct;
}

__device__ __forceinline__ void philox_normals8(uint64_t block, uint64_t image, uint64_t seed,
                                                uint64_t step, float (&z)[8]) {
    uint64_t c[4] = {block, image, 0ull, 0ull};
    philox4x64_10(c, seed, step);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float r = __builtin_amdgcn_sqrtf(-2.0f * ln_uniform((uint32_t)c[k]));
        // the hardware sine and cosine take their argument in turns: 2 pi u2
        const float u2 = fmaf((float)(uint32_t)(c[k] >> 32), 0x1p-32f, 0x1p-33f);
        z[2 * k] = r * __builtin_amdgcn_cosf(u2);
        z[2 * k + 1] = r * __builtin_amdgcn_sinf(u2);
    }
}

__device__ __forceinline__ void accum(float &num, float &den, float c, float u) {
    num += fabsf(c - u);
    den += fabsf(u);
}

__device__ __forceinline__ float update(float x, float c, float u, float w, float c_x, float c_e) {
    return fmaf(c_x, x, c_e * fmaf(w, c - u, u));
}

// Barrier for the LDS exchanges of the reduction only: LDS writes complete,
// then s_barrier -- unlike __syncthreads it does not wait for this
// wavefront's global stores and loads in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

enum Noise { kNoNoise = 0, kNoiseArray = 1, kNoisePhilox = 2 };

// NOISE adds c_z * z to the update: z read from a caller array shaped like x
// (kNoiseArray) or drawn here (kNoisePhilox).  VEC: 16-byte accesses, items
// of 4 floats (8 with drawn noise: one Philox block).
template <bool UPDATE, bool VEC, int NOISE>
__global__ __launch_bounds__(kThreads) void cfg_step_kernel(
    float *__restrict__ x, const float *__restrict__ g_c, const float *__restrict__ g_u,
    const float *__restrict__ z, int64_t n, float w, float c_x, float c_e, float c_z,
    uint64_t seed, uint64_t step, double *__restrict__ partials, int reduce) {
    const int img = blockIdx.y;
    const int blk = blockIdx.x;
    const int nblk = gridDim.x;
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)img * n;
    float num = 0.f, den = 0.f;

    constexpr int F = NOISE == kNoisePhilox ? 2 : 1;   // float4 per item and array
    constexpr int UN = unroll_of<NOISE>();
    float4 cv[UN][F], uv[UN][F], xv[UN][F], zv[UN][F];
    constexpr int ZN = NOISE == kNoisePhilox ? 8 : 1;
    float zn[UN][ZN];   // drawn noise of the pass's items
    int64_t last = -1;   // item base of this thread's final vector pass
    const int64_t n_items = n / (4 * F);
    const int64_t stride = (int64_t)nblk * kThreads * UN;
    const float4 *c4 = reinterpret_cast<const float4 *>(g_c + base);
    const float4 *u4 = reinterpret_cast<const float4 *>(g_u + base);
    float4 *x4 = reinterpret_cast<float4 *>(x + base);
    const float4 *z4 = reinterpret_cast<const float4 *>(z + (NOISE == kNoiseArray ? base : 0));

    auto load_pass = [&](int64_t i0) {
#pragma unroll
        for (int k = 0; k < UN; ++k) {
            const int64_t i = i0 + (int64_t)k * kThreads;
            if (i < n_items)
#pragma unroll
                for (int f = 0; f < F; ++f) cv[k][f] = c4[i * F + f];
        }
#pragma unroll
        for (int k = 0; k < UN; ++k) {
            const int64_t i = i0 + (int64_t)k * kThreads;
            if (i < n_items)
#pragma unroll
                for (int f = 0; f < F; ++f) uv[k][f] = u4[i * F + f];
        }
        if (UPDATE) {
#pragma unroll
            for (int k = 0; k < UN; ++k) {
                const int64_t i = i0 + (int64_t)k * kThreads;
                if (i < n_items)
#pragma unroll
                    for (int f = 0; f < F; ++f) xv[k][f] = x4[i * F + f];
            }
        }
        if (NOISE == kNoiseArray) {
#pragma unroll
            for (int k = 0; k < UN; ++k) {
                const int64_t i = i0 + (int64_t)k * kThreads;
                if (i < n_items) zv[k][0] = z4[i];
            }
        }
        if constexpr (NOISE == kNoisePhilox && UPDATE) {
            // independent of the loads: drawn while they are in flight
#pragma unroll
            for (int k = 0; k < UN; ++k)
                philox_normals8((uint64_t)(i0 + (int64_t)k * kThreads), (uint64_t)img, seed,
                                step, zn[k]);
        }
    };
    auto accum_pass = [&](int64_t i0) {
#pragma unroll
        for (int k = 0; k < UN; ++k) {
            const int64_t i = i0 + (int64_t)k * kThreads;
            if (i < n_items)
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    accum(num, den, cv[k][f].x, uv[k][f].x);
                    accum(num, den, cv[k][f].y, uv[k][f].y);
                    accum(num, den, cv[k][f].z, uv[k][f].z);
                    accum(num, den, cv[k][f].w, uv[k][f].w);
                }
        }
    };
    auto update_pass = [&](int64_t i0) {
#pragma unroll
        for (int k = 0; k < UN; ++k) {
            const int64_t i = i0 + (int64_t)k * kThreads;
            if (i >= n_items) continue;
            float zz[4 * F];
            if constexpr (NOISE == kNoisePhilox) {
#pragma unroll
                for (int e = 0; e < 4 * F; ++e) zz[e] = zn[k][e];
            } else if constexpr (NOISE == kNoiseArray) {
                zz[0] = zv[k][0].x;
                zz[1] = zv[k][0].y;
                zz[2] = zv[k][0].z;
                zz[3] = zv[k][0].w;
            }
#pragma unroll
            for (int f = 0; f < F; ++f) {
                float4 r;
                r.x = update(xv[k][f].x, cv[k][f].x, uv[k][f].x, w, c_x, c_e);
                r.y = update(xv[k][f].y, cv[k][f].y, uv[k][f].y, w, c_x, c_e);
                r.z = update(xv[k][f].z, cv[k][f].z, uv[k][f].z, w, c_x, c_e);
                r.w = update(xv[k][f].w, cv[k][f].w, uv[k][f].w, w, c_x, c_e);
                if (NOISE != kNoNoise) {
                    r.x = fmaf(c_z, zz[4 * f], r.x);
                    r.y = fmaf(c_z, zz[4 * f + 1], r.y);
                    r.z = fmaf(c_z, zz[4 * f + 2], r.z);
                    r.w = fmaf(c_z, zz[4 * f + 3], r.w);
                }
                x4[i * F + f] = r;
            }
        }
    };

    if (VEC) {
        // every pass but the last updates x right away; the last pass's x is
        // written after this workgroup has stored its partial
        for (int64_t i0 = (int64_t)blk * kThreads * UN + tid; i0 < n_items; i0 += stride) {
            load_pass(i0);
            accum_pass(i0);
            if (i0 + stride < n_items || !reduce) {
                if (UPDATE) update_pass(i0);
            } else {
                last = i0;
            }
        }
    } else {
        // unaligned or ragged: one element at a time (a Philox block per 8)
        const float *xs = x + base;
        const float *cs = g_c + base;
        const float *us = g_u + base;
        constexpr int SW = NOISE == kNoisePhilox ? 8 : 1;
        const int64_t nb = (n + SW - 1) / SW;
        for (int64_t j = (int64_t)blk * kThreads + tid; j < nb; j += (int64_t)nblk * kThreads) {
            float zb[8];
            if (UPDATE && NOISE == kNoisePhilox)
                philox_normals8((uint64_t)j, (uint64_t)img, seed, step, zb);
#pragma unroll
            for (int e = 0; e < SW; ++e) {
                const int64_t i = j * SW + e;
                if (i >= n) break;
                const float c = cs[i], u = us[i];
                accum(num, den, c, u);
                if (UPDATE) {
                    float r = update(xs[i], c, u, w, c_x, c_e);
                    if (NOISE == kNoiseArray) r = fmaf(c_z, z[base + i], r);
                    if (NOISE == kNoisePhilox) r = fmaf(c_z, zb[e], r);
                    x[base + i] = r;
                }
            }
        }
    }

    if (!reduce) return;

    // workgroup partial: wave sums (fp32), then the waves in fp64; stored
    // before the last pass's x, which is still to be written
    __shared__ float wnum[kWaves], wden[kWaves];
    num = dfp::wave_sum(num);
    den = dfp::wave_sum(den);
    const int wave = tid / dfp::kWave, lane = tid % dfp::kWave;
    if (lane == 0) {
        wnum[wave] = num;
        wden[wave] = den;
    }
    lds_barrier();
    if (tid == 0) {
        double pn = 0.0, pd = 0.0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            pn += (double)wnum[k];
            pd += (double)wden[k];
        }
        double *slot = partials + 2 * ((int64_t)img * nblk + blk);
        slot[0] = pn;
        slot[1] = pd;
    }
    if (UPDATE && last >= 0) update_pass(last);
}

// Second launch: one wavefront per image sums the image's workgroup partials
// in a fixed order (fp64) and writes the ratio.  The launch boundary orders
// it after every partial store of the first launch.  Lane l adds partials
// l, l + 64, ... in order, with up to kMergeLoads of them loaded at once,
// then a fixed butterfly combines the lanes.
constexpr int kMergeLoads = 8;
__global__ __launch_bounds__(dfp::kWave) void cfg_merge_kernel(const double *__restrict__ partials,
                                                               int nblk, float *__restrict__ out) {
    const int img = blockIdx.x, lane = threadIdx.x;
    const double2 *p = reinterpret_cast<const double2 *>(partials) + (int64_t)img * nblk;
    double a = 0.0, b = 0.0;
    for (int k0 = lane; k0 < nblk; k0 += dfp::kWave * kMergeLoads) {
        double2 v[kMergeLoads];
#pragma unroll
        for (int j = 0; j < kMergeLoads; ++j) {
            const int k = k0 + j * dfp::kWave;
            v[j] = k < nblk ? p[k] : make_double2(0.0, 0.0);
        }
#pragma unroll
        for (int j = 0; j < kMergeLoads; ++j) {
            a += v[j].x;
            b += v[j].y;
        }
    }
    a = dfp::wave_sum(a);
    b = dfp::wave_sum(b);
    if (lane == 0) out[img] = (float)(a / b);
}

// Fill z with the draw the fused step uses (same device code).
__global__ __launch_bounds__(kThreads) void philox_normal_kernel(float *__restrict__ z, int64_t n,
                                                                 uint64_t seed, uint64_t step) {
    const int img = blockIdx.y;
    const int64_t nb = (n + 7) / 8;
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < nb;
         j += (int64_t)gridDim.x * kThreads) {
        float zb[8];
        philox_normals8((uint64_t)j, (uint64_t)img, seed, step, zb);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (j * 8 + e < n) z[(int64_t)img * n + j * 8 + e] = zb[e];
    }
}

// Raw Philox4x64-10 words of counters (j, c1, 0, 0), j < blocks, key (k0, k1).
__global__ __launch_bounds__(kThreads) void philox_raw_kernel(uint64_t *__restrict__ out,
                                                              int64_t blocks, uint64_t c1,
                                                              uint64_t k0, uint64_t k1) {
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < blocks;
         j += (int64_t)gridDim.x * kThreads) {
        uint64_t c[4] = {(uint64_t)j, c1, 0ull, 0ull};
        philox4x64_10(c, k0, k1);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[j * 4 + e] = c[e];
    }
}

size_t workspace_need(int64_t n_per_image, int batch) {
    // items of 4 floats need the most workgroups
    return (size_t)batch * plan_blocks(n_per_image, 4) * 2 * sizeof(double);
}

struct NoiseArgs {
    int kind;
    const float *z;
    float c_z;
    uint64_t seed, step;
};

template <bool UPDATE>
dfp_status launch(float *x, const float *g_c, const float *g_u, const NoiseArgs &nz, int64_t n,
                  int batch, float w, float c_x, float c_e, float *out, void *ws, size_t ws_bytes,
                  hipStream_t stream) {
    if (!g_c || !g_u || (UPDATE && !x) || n <= 0 || batch <= 0 || batch > 65535)
        return DFP_ERR_INVALID_ARG;
    const int reduce = out != nullptr;
    if (reduce && (!ws || ws_bytes < workspace_need(n, batch) ||
                   (reinterpret_cast<uintptr_t>(ws) % 16) != 0))
        return DFP_ERR_INVALID_ARG;
    const int item = nz.kind == kNoisePhilox ? 8 : 4;
    const bool vec = (n % item == 0) && (reinterpret_cast<uintptr_t>(g_c) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(g_u) % 16 == 0) &&
                     (!UPDATE || reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                     (nz.kind != kNoiseArray || reinterpret_cast<uintptr_t>(nz.z) % 16 == 0);
    double *partials = reduce ? static_cast<double *>(ws) : nullptr;
    // the workspace holds partials for plan_blocks(n, 4) workgroups per image
    dim3 grid((unsigned)plan_blocks(n, item, nz.kind == kNoisePhilox ? 1 : kUnroll),
              (unsigned)batch);
#define DFP_CFG_LAUNCH(V, N)                                                                  \
    hipLaunchKernelGGL((cfg_step_kernel<UPDATE, V, N>), grid, dim3(kThreads), 0, stream, x,    \
                       g_c, g_u, nz.z, n, w, c_x, c_e, nz.c_z, nz.seed, nz.step, partials,    \
                       reduce)
    if (nz.kind == kNoiseArray) {
        if (vec) DFP_CFG_LAUNCH(true, kNoiseArray);
        else DFP_CFG_LAUNCH(false, kNoiseArray);
    } else if (nz.kind == kNoisePhilox) {
        if (vec) DFP_CFG_LAUNCH(true, kNoisePhilox);
        else DFP_CFG_LAUNCH(false, kNoisePhilox);
    } else {
        if (vec) DFP_CFG_LAUNCH(true, kNoNoise);
        else DFP_CFG_LAUNCH(false, kNoNoise);
    }
#undef DFP_CFG_LAUNCH
    if (reduce)
        hipLaunchKernelGGL(cfg_merge_kernel, dim3((unsigned)batch), dim3(dfp::kWave), 0, stream,
                           partials, (int)grid.x, out);
    return dfp::launch_status();
}

}  // namespace

size_t dfp_cfg_workspace_bytes(int64_t n_per_image, int batch) {
    if (n_per_image <= 0 || batch <= 0) return 0;
    return workspace_need(n_per_image, batch);
}

extern "C" dfp_status dfp_cfg_step(float *x, const float *g_c, const float *g_u,
                                   int64_t n_per_image, int batch, float w, double c_x,
                                   double c_e, float *relmae_out, void *workspace,
                                   size_t ws_bytes, hipStream_t stream) {
    if (!std::isfinite(w) || !std::isfinite(c_x) || !std::isfinite(c_e))
        return DFP_ERR_INVALID_ARG;
    const NoiseArgs nz{kNoNoise, nullptr, 0.f, 0, 0};
    return launch<true>(x, g_c, g_u, nz, n_per_image, batch, w, (float)c_x, (float)c_e,
                        relmae_out, workspace, ws_bytes, stream);
}

extern "C" dfp_status dfp_cfg_step_noise(float *x, const float *g_c, const float *g_u,
                                         const float *z, int64_t n_per_image, int batch, float w,
                                         double c_x, double c_e, double c_z, float *relmae_out,
                                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!z || !std::isfinite(w) || !std::isfinite(c_x) || !std::isfinite(c_e) ||
        !std::isfinite(c_z))
        return DFP_ERR_INVALID_ARG;
    const NoiseArgs nz{kNoiseArray, z, (float)c_z, 0, 0};
    return launch<true>(x, g_c, g_u, nz, n_per_image, batch, w, (float)c_x, (float)c_e,
                        relmae_out, workspace, ws_bytes, stream);
}

extern "C" dfp_status dfp_cfg_step_philox(float *x, const float *g_c, const float *g_u,
                                          int64_t n_per_image, int batch, float w, double c_x,
                                          double c_e, double c_z, uint64_t seed, uint64_t step,
                                          float *relmae_out, void *workspace, size_t ws_bytes,
                                          hipStream_t stream) {
    if (!std::isfinite(w) || !std::isfinite(c_x) || !std::isfinite(c_e) || !std::isfinite(c_z))
        return DFP_ERR_INVALID_ARG;
    const NoiseArgs nz{kNoisePhilox, nullptr, (float)c_z, seed, step};
    return launch<true>(x, g_c, g_u, nz, n_per_image, batch, w, (float)c_x, (float)c_e,
                        relmae_out, workspace, ws_bytes, stream);
}

// ------------------------------------------------------ no-allocation step
// Scratch of dfp_cfg_step_static: the per-workgroup rel-MAE partials in a
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never uses this name as an address: each device's copy is found
// with hipGetSymbolAddress on the first call on that device.
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
static __device__ __align__(256) double scratch[kStaticScratchBytes / sizeof(double)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
dfp_status static_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DFP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DFP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFP_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DFP_OK;
}

extern "C" size_t dfp_cfg_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" dfp_status dfp_cfg_step_static(float *x, const float *g_c, const float *g_u,
                                          int64_t n_per_image, int batch, float w, double c_x,
                                          double c_e, float *relmae_out, hipStream_t stream) {
    if (!std::isfinite(w) || !std::isfinite(c_x) || !std::isfinite(c_e))
        return DFP_ERR_INVALID_ARG;
    if (!x || !g_c || !g_u || n_per_image <= 0 || batch <= 0 || batch > 65535)
        return DFP_ERR_INVALID_ARG;
    void *ws = nullptr;
    if (relmae_out) {
        if (workspace_need(n_per_image, batch) > kStaticScratchBytes) return DFP_ERR_TOO_LARGE;
        const dfp_status st = static_scratch(&ws);
        if (st != DFP_OK) return st;
    }
    const NoiseArgs nz{kNoNoise, nullptr, 0.f, 0, 0};
    return launch<true>(x, g_c, g_u, nz, n_per_image, batch, w, (float)c_x, (float)c_e,
                        relmae_out, ws, relmae_out ? kStaticScratchBytes : 0, stream);
}

extern "C" dfp_status dfp_relmae(const float *g_c, const float *g_u, int64_t n_per_image,
                                 int batch, float *out, void *workspace, size_t ws_bytes,
                                 hipStream_t stream) {
    if (!out) return DFP_ERR_INVALID_ARG;
    const NoiseArgs nz{kNoNoise, nullptr, 0.f, 0, 0};
    return launch<false>(nullptr, g_c, g_u, nz, n_per_image, batch, 0.f, 0.f, 0.f, out,
                         workspace, ws_bytes, stream);
}

extern "C" dfp_status dfp_philox_normal(float *z, int64_t n_per_image, int batch, uint64_t seed,
                                        uint64_t step, hipStream_t stream) {
    if (!z || n_per_image <= 0 || batch <= 0 || batch > 65535) return DFP_ERR_INVALID_ARG;
    const int64_t nb = (n_per_image + 7) / 8;
    int64_t blocks = (nb + kThreads - 1) / kThreads;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    hipLaunchKernelGGL(philox_normal_kernel, dim3((unsigned)blocks, (unsigned)batch),
                       dim3(kThreads), 0, stream, z, n_per_image, seed, step);
    return dfp::launch_status();
}

extern "C" dfp_status dfp_philox4x64_10(uint64_t *out, int64_t blocks, uint64_t counter1,
                                        uint64_t key0, uint64_t key1, hipStream_t stream) {
    if (blocks < 0 || (blocks > 0 && !out)) return DFP_ERR_INVALID_ARG;
    if (blocks == 0) return DFP_OK;
    int64_t g = (blocks + kThreads - 1) / kThreads;
    if (g > kMaxBlocks) g = kMaxBlocks;
    hipLaunchKernelGGL(philox_raw_kernel, dim3((unsigned)g), dim3(kThreads), 0, stream, out,
                       blocks, counter1, key0, key1);
    return dfp::launch_status();
}
